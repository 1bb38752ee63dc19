"""Properties of the compiled gfx950 code that the sources rely on (CPU only:
hipcc cross-compiles to assembly, nothing runs).

- No kernel writes through the scalar data cache (scalar stores, scalar
  atomics, scalar cache write-back): every store and atomic is a vector one.
- The direct-to-LDS loads set M0 in inline assembly; that is only sound while
  the compiler itself keeps nothing in M0 in those kernels.
"""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sample_gradient_clipping_layer_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _asm(src):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                          "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
                          "-S", "-o", "-", src], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    return out.stdout


SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
    os.path.join(ROOT, "sample_gradient_clipping_layer_amd", "ceilings", "dp_ceilings.hip")]


@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_no_scalar_memory_writes(src):
    asm = _asm(src)
    bad = re.findall(r"^\s*(s_store\w*|s_buffer_store\w*|s_scratch_store\w*|s_atomic\w*|s_buffer_atomic\w*|"
                     r"s_dcache_wb\w*|s_dcache_discard\w*)\b", asm, flags=re.M)
    assert not bad, sorted(set(bad))


def test_m0_only_set_for_lds_dma():
    asm = _asm(os.path.join(CSRC, "dp_contract.hip"))
    lines = [l.strip() for l in asm.splitlines() if re.search(r"\bm0\b", l) and not l.strip().startswith(";")]
    assert lines, "expected the direct-to-LDS loads"
    # the direct-to-LDS asm sets m0 from a scalar register (any SGPR, vcc halves included)
    other = [l for l in lines if not re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", l)]
    assert not other, other[:5]
