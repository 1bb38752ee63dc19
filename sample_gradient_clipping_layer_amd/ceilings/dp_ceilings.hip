// Hardware ceilings of the instruction mixes the clipping kernels are built
// from, measured on every CU of the GPU: the price list that the kernels'
// roofline fractions are read against.
//
// Each probe runs one 512-thread workgroup per CU (8 waves, 2 per SIMD: the
// occupancy of the direct-to-LDS kernels), 1024 workgroups, a fixed number of
// iterations of one instruction pattern, and reports a rate:
// - mfma_const / mfma_random: v_mfma_f32_32x32x16_bf16 on 4 independent
//   accumulators, operands constant or random bf16 (sign, mantissa and a
//   2-bit exponent spread). The matrix cores draw more power on toggling
//   data and the clock drops; the random-data rate is the practical peak.
// - lds_b128 / lds_tr_b16: ds_read_b128 and ds_read_b64_tr_b16 only, in
//   bytes per clock per CU at the nominal 2.4 GHz.
// - dma_l2: global_load_lds_dwordx4 (16 bytes per lane straight into LDS)
//   from a 2 MiB buffer that stays in L2, bytes per clock per CU.
// - mix_gram: the long-sequence ghost kernel's chunk without its barrier and
//   loads: 16 ds_read_b128 then 16 MFMAs per wave and iteration (random data).
// - mix_gram_dma: the same plus 6 direct-to-LDS loads per wave and iteration
//   (its load-to-read byte ratio), not waited on by the reads.
// - mix_contract: the bf16 contraction's k-step: 6 operand fragments from
//   12 ds_read_b64_tr_b16 and 8 MFMAs (random data).
// - mix_contract_pipe: the same with the next k-step's 12 reads issued ahead
//   of this k-step's MFMAs.
// - mix_contract_dma: mix_contract plus 2 direct-to-LDS loads per wave and
//   k-step (the 256 x 256 tile's load-to-read byte ratio), not waited on by
//   the reads.
// - hbm_rows / hbm_contiguous: HBM read rate of one workgroup per CU reading
//   blocks of 128 rows x 1536 bytes (one sample's rows of a 768-feature bf16
//   layer) of a 1.5 GiB buffer, 256-byte slices of every row at a time (the
//   Gram kernels' order), or each block as one contiguous run; 8 loads of 16
//   bytes in flight per thread.
// Every LDS address is masked into the kernel's 96 KB allocation and every
// global offset into the 2 MiB source (1.5 GiB for the HBM probes); each
// thread stores one float.
//
// Build: python -m sample_gradient_clipping_layer_amd._build (writes
// sample_gradient_clipping_layer_amd/dp_ceilings). Run it with no arguments;
// it prints one JSON line.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) unsigned char lds_uchar;

constexpr int kThreads = 512, kBlocks = 1024, kIters = 4096;
constexpr int kLdsBytes = 98304;           // forces one workgroup per CU
constexpr uint32_t kReadMask = 65535;      // reads stay in the first 64 KB
constexpr uint32_t kSrcBytes = 2u << 20;   // global source of the loads
constexpr int64_t kHbmBytes = 1536ll << 20; // source of the HBM probes: past the 256 MB last-level cache
constexpr int kRowBytes = 1536, kRows = 128, kSlice = 256, kHbmUnroll = 8;

enum Mode {
  MFMA_CONST, MFMA_RANDOM, LDS_B128, LDS_TR, DMA_L2, MIX_GRAM, MIX_GRAM_DMA, MIX_CONTRACT, MIX_CONTRACT_PIPE,
  MIX_CONTRACT_DMA, NMODES
};

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ u32x4 rd128(uint32_t a) { return *(const lds_u32x4*)(uintptr_t)(a & kReadMask); }
// one MFMA operand from two transposing 8-byte reads, 2 KB apart
__device__ __forceinline__ u32x4 rdtr(uint32_t a) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a & kReadMask));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)((a + 2048) & kReadMask));
  u32x4 r;
  r[0] = (uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  r[1] = (uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  r[2] = (uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  r[3] = (uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return r;
}
// 16 bytes per lane from src + off into LDS at lds_base + 16 * lane (base in M0)
__device__ __forceinline__ void dma16(const void* src, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(src), "s"(lds_base)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h *= 2654435761u;
  h ^= h >> 15;
  h *= 2246822519u;
  return h ^ (h >> 13);
}
// two bf16 with random sign and mantissa and exponents 124..127 (finite sums)
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t i) {
  const uint32_t h = mix32(i + 1);
  return (h & 0x807F807Fu) | 0x3E003E00u | ((h >> 8) & 0x01800180u);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_probe(const unsigned char* __restrict__ src, float* out) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  uint32_t* l32 = reinterpret_cast<uint32_t*>(lds);
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += kThreads)
    l32[i] = MODE == MFMA_CONST ? 0x3C003C00u : rand_bf16x2((uint32_t)i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t l0 = (uint32_t)reinterpret_cast<uintptr_t>((const lds_uchar*)lds);
  uint32_t rbase = l0 + wave * 4096 + lane * 16;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  u32x4 a0, b0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a0[e] = l32[(lane * 4 + e) & 16383];
    b0[e] = l32[(lane * 4 + 256 + e) & 16383];
  }
  const uint32_t wsrc = (uint32_t)(blockIdx.x * 8 + wave) * 6144u;
  // MIX_CONTRACT_PIPE: this k-step's operands, read in the previous iteration
  u32x4 pa[2], pb[4];
  if constexpr (MODE == MIX_CONTRACT_PIPE) {
#pragma unroll
    for (int i = 0; i < 2; ++i) pa[i] = rdtr(rbase + i * 8192);
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = rdtr(rbase + 32768 + i * 4096);
  }
  for (int it = 0; it < kIters; ++it) {
    asm volatile("" : "+v"(rbase));  // a fresh address each iteration: no read is hoisted
    if constexpr (MODE == DMA_L2 || MODE == MIX_GRAM_DMA || MODE == MIX_CONTRACT_DMA) {
      constexpr int N = MODE == MIX_CONTRACT_DMA ? 2 : 6;
      const uint32_t g0 = wsrc + (uint32_t)it * 49152u;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const uint32_t goff = ((g0 + i * 1024u) & (kSrcBytes - 1) & ~1023u) + lane * 16;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane(((it & 1) * 49152 + wave * 6144 + i * 1024) &
                                                                     ~1023);
        dma16(src, goff, l0 + lo);  // lo + 1 KB <= 96 KB
      }
    }
    if constexpr (MODE == MFMA_CONST || MODE == MFMA_RANDOM) {
      asm volatile("" : "+v"(a0), "+v"(b0));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma(a0, b0, acc[j]);
    } else if constexpr (MODE == LDS_B128) {
      u32x4 f[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = rd128(rbase + i * 1024);
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(f[i]));
    } else if constexpr (MODE == LDS_TR) {
      u32x4 f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = rdtr(rbase + i * 4096);
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(f[i]));
    } else if constexpr (MODE == MIX_GRAM || MODE == MIX_GRAM_DMA) {
      u32x4 fa[4][2], fb[4][2];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          fa[kk][b] = rd128(rbase + kk * 2048 + b * 1024);
          fb[kk][b] = rd128(rbase + 16384 + kk * 2048 + b * 1024);
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj) acc[bi * 2 + bj] = mfma(fa[kk][bi], fb[kk][bj], acc[bi * 2 + bj]);
    } else if constexpr (MODE == MIX_CONTRACT || MODE == MIX_CONTRACT_DMA) {
      u32x4 fa[2], fb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = rdtr(rbase + i * 8192);
#pragma unroll
      for (int i = 0; i < 4; ++i) fb[i] = rdtr(rbase + 32768 + i * 4096);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma(fa[i], fb[j], acc[j]);
    } else if constexpr (MODE == MIX_CONTRACT_PIPE) {
      u32x4 na[2], nb[4];  // the next k-step's operands, in flight during this one's MFMAs
#pragma unroll
      for (int i = 0; i < 2; ++i) na[i] = rdtr(rbase + i * 8192);
#pragma unroll
      for (int i = 0; i < 4; ++i) nb[i] = rdtr(rbase + 32768 + i * 4096);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma(pa[i], pb[j], acc[j]);
#pragma unroll
      for (int i = 0; i < 2; ++i) pa[i] = na[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = nb[i];
    }
    if constexpr (MODE == DMA_L2 || MODE == MIX_GRAM_DMA) wait_vm<12>();  // two iterations of loads in flight
    if constexpr (MODE == MIX_CONTRACT_DMA) wait_vm<4>();
  }
  wait_vm<0>();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// HBM read probe: workgroup b reads block b (kRows rows of kRowBytes) either
// in 256-byte slices of every row at a time (SLICED) or as one run.
template <bool SLICED>
__global__ __launch_bounds__(kThreads, 1) void k_rows(const unsigned char* __restrict__ src, int64_t nblk,
                                                      float* out) {
  extern __shared__ unsigned char unused_lds[];  // one workgroup per CU
  const int64_t blk = blockIdx.x;
  if (blk >= nblk) return;
  const unsigned char* b = src + blk * (int64_t)kRows * kRowBytes;
  constexpr int kPieces = kRows * kRowBytes / 16;  // 16-byte pieces of a block
  constexpr int kPerSlice = kRows * (kSlice / 16);
  u32x4 x = {0u, 0u, 0u, 0u};
  for (int base = 0; base < kPieces; base += kThreads * kHbmUnroll) {
    u32x4 v[kHbmUnroll];
#pragma unroll
    for (int u = 0; u < kHbmUnroll; ++u) {
      const int i = base + u * kThreads + (int)threadIdx.x;  // < kPieces: kPieces % (kThreads * kHbmUnroll) == 0
      int off = i * 16;
      if constexpr (SLICED) {
        const int sl = i / kPerSlice, r = (i % kPerSlice) / (kSlice / 16), pc = i % (kSlice / 16);
        off = r * kRowBytes + sl * kSlice + pc * 16;
      }
      v[u] = *reinterpret_cast<const u32x4*>(b + off);
    }
#pragma unroll
    for (int u = 0; u < kHbmUnroll; ++u) x ^= v[u];
  }
  out[blk * kThreads + threadIdx.x] = (float)(x[0] ^ x[1] ^ x[2] ^ x[3]);
}
static_assert((kRows * kRowBytes / 16) % (kThreads * kHbmUnroll) == 0 && kRowBytes % kSlice == 0, "whole passes");

template <bool SLICED>
int time_rows(const unsigned char* src, float* out, double* seconds) {
  const int64_t nblk = kHbmBytes / ((int64_t)kRows * kRowBytes);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rows<SLICED>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  hipLaunchKernelGGL(k_rows<SLICED>, dim3((unsigned)nblk), dim3(kThreads), kLdsBytes, 0, src, nblk, out);
  const int reps = 5;
  hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(k_rows<SLICED>, dim3((unsigned)nblk), dim3(kThreads), kLdsBytes, 0, src, nblk, out);
  hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  *seconds = ms * 1e-3 / reps;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int MODE>
int time_mode(const unsigned char* src, float* out, double* seconds) {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_probe<MODE>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  hipLaunchKernelGGL(k_probe<MODE>, dim3(kBlocks), dim3(kThreads), kLdsBytes, 0, src, out);  // warm-up
  const int reps = 5;
  hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(k_probe<MODE>, dim3(kBlocks), dim3(kThreads), kLdsBytes, 0, src, out);
  hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  *seconds = ms * 1e-3 / reps;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int main() {
  unsigned char* src = nullptr;
  unsigned char* big = nullptr;
  float* out = nullptr;
  const int64_t nblk = kHbmBytes / ((int64_t)kRows * kRowBytes);
  const size_t nout = (size_t)(nblk > kBlocks ? nblk : kBlocks) * kThreads;
  if (hipMalloc(&src, kSrcBytes) != hipSuccess || hipMalloc(&big, kHbmBytes) != hipSuccess ||
      hipMalloc(&out, nout * 4) != hipSuccess || hipMemset(src, 0x3C, kSrcBytes) != hipSuccess ||
      hipMemset(big, 0x3C, kHbmBytes) != hipSuccess) {
    fprintf(stderr, "dp_ceilings: device allocation failed\n");
    return 1;
  }
  double t[NMODES] = {}, t_rows = 0.0, t_run = 0.0;
  int err = time_mode<MFMA_CONST>(src, out, &t[MFMA_CONST]) | time_mode<MFMA_RANDOM>(src, out, &t[MFMA_RANDOM]) |
            time_mode<LDS_B128>(src, out, &t[LDS_B128]) | time_mode<LDS_TR>(src, out, &t[LDS_TR]) |
            time_mode<DMA_L2>(src, out, &t[DMA_L2]) | time_mode<MIX_GRAM>(src, out, &t[MIX_GRAM]) |
            time_mode<MIX_GRAM_DMA>(src, out, &t[MIX_GRAM_DMA]) | time_mode<MIX_CONTRACT>(src, out, &t[MIX_CONTRACT]) |
            time_mode<MIX_CONTRACT_PIPE>(src, out, &t[MIX_CONTRACT_PIPE]) |
            time_mode<MIX_CONTRACT_DMA>(src, out, &t[MIX_CONTRACT_DMA]) | time_rows<true>(big, out, &t_rows) |
            time_rows<false>(big, out, &t_run);
  if (err || hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "dp_ceilings: a probe failed\n");
    return 1;
  }
  const double waves = (double)kBlocks * kThreads / 64, cu_clk = 256 * 2.4e9, peak = 2.5e15;
  const double fl16 = waves * kIters * 16 * 32768.0, fl8 = waves * kIters * 8 * 32768.0;
  const double hbm = (double)nblk * kRows * kRowBytes;
  auto tf = [](double fl, double s) { return fl / s / 1e12; };
  printf("{\"probe\": \"dp_ceilings\", \"waves_per_cu\": 8, \"nominal_clock_ghz\": 2.4, \"bf16_peak_tflops\": 2500, "
         "\"mfma_const_tflops\": %.0f, \"mfma_random_tflops\": %.0f, \"mfma_random_frac\": %.3f, "
         "\"lds_b128_bytes_per_clk_cu\": %.1f, \"lds_tr_b16_bytes_per_clk_cu\": %.1f, \"dma_l2_bytes_per_clk_cu\": %.1f, "
         "\"mix_gram_tflops\": %.0f, \"mix_gram_dma_tflops\": %.0f, \"mix_contract_tflops\": %.0f, "
         "\"mix_contract_frac\": %.3f, \"mix_contract_pipe_tflops\": %.0f, \"mix_contract_pipe_frac\": %.3f, "
         "\"mix_contract_dma_tflops\": %.0f, \"mix_contract_dma_frac\": %.3f, \"hbm_rows_256B_tbs\": %.2f, "
         "\"hbm_contiguous_tbs\": %.2f}\n",
         tf(fl16, t[MFMA_CONST]), tf(fl16, t[MFMA_RANDOM]), tf(fl16, t[MFMA_RANDOM]) * 1e12 / peak,
         waves * kIters * 16 * 1024 / t[LDS_B128] / cu_clk, waves * kIters * 16 * 512 / t[LDS_TR] / cu_clk,
         waves * kIters * 6144 / t[DMA_L2] / cu_clk, tf(fl16, t[MIX_GRAM]), tf(fl16, t[MIX_GRAM_DMA]),
         tf(fl8, t[MIX_CONTRACT]), tf(fl8, t[MIX_CONTRACT]) * 1e12 / peak, tf(fl8, t[MIX_CONTRACT_PIPE]),
         tf(fl8, t[MIX_CONTRACT_PIPE]) * 1e12 / peak, tf(fl8, t[MIX_CONTRACT_DMA]),
         tf(fl8, t[MIX_CONTRACT_DMA]) * 1e12 / peak, hbm / t_rows / 1e12, hbm / t_run / 1e12);
  hipFree(src);
  hipFree(big);
  hipFree(out);
  return 0;
}
