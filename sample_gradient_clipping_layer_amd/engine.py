"""Privacy engine front end: per-sample clipping and Gaussian noise for the
Linear and Conv2d layers of a torch model, through the C ABI.

"Scalable and Efficient Training of Large CNNs with DP", App. E (the privacy
engine with its 'ghost' and 'ghost-mixed' modes) and Sec. 3 (ghost norm, then
the weighted gradient instead of per-sample gradients): hooks keep each
layer's input a and output gradient dL/ds during one ordinary forward and
backward pass of the summed per-sample loss; step() then runs the library's
path over all layers -- the per-sample norm over every layer, the clip
factors, and each layer's clipped noised mean -- and writes the results into
the parameters' .grad. A convolution's input is unfolded into U(a) (same
page, Sec. 2.2: D = C_in * kH * kW features per output position) by the
library (dp_unfold2d), and the conv layers share the multi-layer calls with
the linear ones; with conv_input="folded" the library instead forms U(a)'s
rows inside its kernels (dp_conv_* calls, one per layer; nothing unfolded is
stored), and with conv_input="unfolded" torch unfolds each input (at
ResNet-18 shapes torch's unfold alone takes several times the whole
clipping path).

Only argument marshalling and layout changes happen here; every step of the
clipping path runs in libdpclip.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

from . import (DP_BF16, DP_F32, MODE_EXPLICIT, MODE_GHOST, MODE_MIXED, MODE_TIME, conv_geometry, dp_clip_factors,
               dp_clipped_sum_noise_layers, dp_conv_clipped_sum_noise, dp_conv_norm, dp_conv_workspace_bytes,
               dp_ghost_norm_clip_layers, dp_ghost_norm_layers, dp_layers_workspace_bytes, dp_unfold2d)

MODES = {"ghost-mixed": MODE_MIXED, "ghost": MODE_GHOST, "explicit": MODE_EXPLICIT, "time": MODE_TIME}


class _Layer:
    def __init__(self, module: torch.nn.Module):
        self.module = module
        self.a = None   # the module's input of the last forward pass
        self.g = None   # dL/d(output) of the last backward pass


class PrivacyEngine:
    """Flat (global) per-sample clipping at bound C with noise multiplier
    sigma for every nn.Linear and nn.Conv2d (groups = 1) with trainable
    parameters in `model`.

    Usage, per step:
        out = model(x)                       # hooks keep the layer inputs
        per_sample_loss(out, y).sum().backward()   # hooks keep dL/ds
        engine.step(step_index)              # .grad = (sum_i c_i g_i + N(0, s^2 C^2 I)) / B

    The backward pass must be of the SUM of the per-sample losses, so that the
    kept output gradients are the per-sample ones. A module may run once per
    forward pass. Any other trainable parameter makes the constructor fail:
    its per-sample gradient would go unclipped.

    mode: the per-layer path rule ('ghost-mixed', 'ghost', 'explicit',
    'time'). conv_input: 'library-unfold' (the default: the library writes
    each Conv2d input's unfolding, and the layers share the multi-layer
    calls), 'folded' (the library takes each Conv2d input as it is and forms
    the unfolded rows in its kernels, one call per Conv2d layer; no unfolded
    copy in memory) or 'unfolded' (torch unfolds each Conv2d input).
    """

    def __init__(self, model: torch.nn.Module, C: float, sigma: float, seed: int = 0, mode: str = "ghost-mixed",
                 kappa: int = 1, conv_input: str = "library-unfold"):
        if mode not in MODES:
            raise ValueError(f"mode must be one of {sorted(MODES)}")
        if conv_input not in ("library-unfold", "unfolded", "folded"):
            raise ValueError("conv_input must be 'library-unfold', 'unfolded' or 'folded'")
        self.folded = conv_input == "folded"
        self.library_unfold = conv_input == "library-unfold"
        self.C, self.sigma, self.seed = float(C), float(sigma), int(seed)
        self.mode, self.kappa = MODES[mode], int(kappa)
        self.layers: list[_Layer] = []
        covered = set()
        for m in model.modules():
            if isinstance(m, (torch.nn.Linear, torch.nn.Conv2d)) and any(p.requires_grad for p in m.parameters()):
                if isinstance(m, torch.nn.Conv2d) and m.groups != 1:
                    raise ValueError("Conv2d with groups != 1 is not supported")
                if isinstance(m, torch.nn.Conv2d) and m.padding_mode != "zeros":
                    raise ValueError("Conv2d padding must be zeros")
                if isinstance(m, torch.nn.Conv2d) and isinstance(m.padding, str) and m.padding != "valid":
                    raise ValueError("Conv2d padding must be numeric or 'valid'")
                if not m.weight.requires_grad:
                    raise ValueError("a layer with a trainable bias needs a trainable weight (one norm covers both)")
                self.layers.append(_Layer(m))
                covered.update(id(p) for p in m.parameters())
        others = [n for n, p in model.named_parameters() if p.requires_grad and id(p) not in covered]
        if others:
            raise ValueError(f"trainable parameters outside Linear/Conv2d layers: {others}")
        if not self.layers:
            raise ValueError("no Linear or Conv2d layer with trainable parameters")
        self._handles = []
        for L in self.layers:
            self._handles.append(L.module.register_forward_hook(self._forward_hook(L)))
            self._handles.append(L.module.register_full_backward_hook(self._backward_hook(L)))
        self.last_norms = None  # per-sample norms of the last step

    @staticmethod
    def _forward_hook(L):
        def hook(module, inputs, output):
            if L.a is not None and L.g is None:
                raise RuntimeError("a module ran twice in one forward pass")
            L.a = inputs[0].detach()
            L.g = None
        return hook

    @staticmethod
    def _backward_hook(L):
        def hook(module, grad_input, grad_output):
            L.g = grad_output[0].detach()
        return hook

    def detach(self):
        """Remove the hooks."""
        for h in self._handles:
            h.remove()
        self._handles = []

    @staticmethod
    def _padding(m):
        return 0 if isinstance(m.padding, str) else m.padding  # 'valid' is no padding

    def _is_folded(self, L):
        return self.folded and isinstance(L.module, torch.nn.Conv2d)

    def _operands(self, L):
        """(A [B, T, d], G [B, T, p]) of one layer, contiguous, in the activation dtype;
        for a conv layer taken folded, (a [B, C_in, H, W], G [B, T, p], geometry)."""
        m, a, g = L.module, L.a, L.g
        if a is None or g is None:
            raise RuntimeError("step() needs one forward and one backward pass of every layer first")
        B = a.shape[0]
        dt = a.dtype if a.dtype in (torch.float32, torch.bfloat16) else torch.float32
        if isinstance(m, torch.nn.Linear):
            A = a.reshape(B, -1, a.shape[-1])
            G = g.reshape(B, -1, g.shape[-1])
        elif self._is_folded(L):
            geo = conv_geometry(a.shape[1], a.shape[2], a.shape[3], m.kernel_size, m.stride, self._padding(m),
                                m.dilation)
            G = g.reshape(B, g.shape[1], -1).transpose(1, 2)
            return a.to(dt).contiguous(), G.to(dt).contiguous(), geo
        elif self.library_unfold:
            geo = conv_geometry(a.shape[1], a.shape[2], a.shape[3], m.kernel_size, m.stride, self._padding(m),
                                m.dilation)
            A = dp_unfold2d(a.to(dt).contiguous(), geo)  # [B, T, D], written by the library
            G = g.reshape(B, g.shape[1], -1).transpose(1, 2)
        else:
            U = F.unfold(a, m.kernel_size, dilation=m.dilation, padding=self._padding(m), stride=m.stride)  # [B, D, L]
            A = U.transpose(1, 2)
            G = g.reshape(B, g.shape[1], -1).transpose(1, 2)
        return A.to(dt).contiguous(), G.to(dt).contiguous()

    def step(self, step: int, denom: float | None = None):
        """Clipped noised mean gradients into .grad; returns the per-sample norms.

        The noise stream of a layer is its index in the engine's layer list
        (the model's module order), whichever call serves it."""
        ops = [self._operands(L) for L in self.layers]
        B = ops[0][0].shape[0]
        dev = ops[0][0].device
        dtypes = {op[0].dtype for op in ops}
        if len(dtypes) != 1:
            raise RuntimeError("all layers must share one activation dtype")
        dt = DP_BF16 if ops[0][0].dtype == torch.bfloat16 else DP_F32
        denom = float(B) if denom is None else float(denom)
        has_bias = [L.module.bias is not None and L.module.bias.requires_grad for L in self.layers]
        dense = [k for k, op in enumerate(ops) if len(op) == 2]   # [B, T, d] operands: multi-layer calls
        folded = [k for k, op in enumerate(ops) if len(op) == 3]  # folded conv inputs: dp_conv_* calls
        sq = torch.empty(B, dtype=torch.float32, device=dev)
        c = torch.empty(B, dtype=torch.float32, device=dev)
        norms = torch.empty(B, dtype=torch.float32, device=dev)
        ws = None
        if dense:
            dops, dhb = [ops[k] for k in dense], [has_bias[k] for k in dense]
            ws = torch.empty(max(256, dp_layers_workspace_bytes(dops, has_bias=dhb, mode=self.mode,
                                                                kappa=self.kappa)), dtype=torch.uint8, device=dev)
            if folded:
                dp_ghost_norm_layers(dops, sq, has_bias=dhb, mode=self.mode, kappa=self.kappa, workspace=ws)
            else:  # every layer in this call: its kernels form the clip factors too (the same bits)
                dp_ghost_norm_clip_layers(dops, sq, self.C, c, norms, has_bias=dhb, mode=self.mode,
                                          kappa=self.kappa, workspace=ws)
        wsc = {}
        for k in folded:
            a, G, geo = ops[k]
            wsc[k] = torch.empty(max(256, dp_conv_workspace_bytes(geo, dt, B, G.shape[2], has_bias[k], self.mode,
                                                                  self.kappa)), dtype=torch.uint8, device=dev)
            dp_conv_norm(a, G, geo, sq, has_bias=has_bias[k], mode=self.mode, kappa=self.kappa,
                         accumulate=bool(dense) or k != folded[0], workspace=wsc[k])
        if folded:
            dp_clip_factors(sq, self.C, c, norms)
        d_of = [op[2].C_in * op[2].kh * op[2].kw if len(op) == 3 else op[0].shape[2] for op in ops]
        outs = [torch.empty(d_of[k], op[1].shape[2], dtype=torch.float32, device=dev) for k, op in enumerate(ops)]
        bouts = [torch.empty(op[1].shape[2], dtype=torch.float32, device=dev) if hb else None
                 for op, hb in zip(ops, has_bias)]
        if dense:
            dp_clipped_sum_noise_layers([ops[k] for k in dense], c, self.C, self.sigma, denom, self.seed, step,
                                        [outs[k] for k in dense],
                                        bias_outs=[bouts[k] for k in dense] if any(dhb) else None, has_bias=dhb,
                                        layer_ids=dense, workspace=ws)
        for k in folded:
            a, G, geo = ops[k]
            dp_conv_clipped_sum_noise(a, G, geo, c, self.C, self.sigma, denom, self.seed, k, step, outs[k],
                                      bias_out=bouts[k], workspace=wsc[k])
        for L, out, bout in zip(self.layers, outs, bouts):
            w = L.module.weight
            if w.requires_grad:
                w.grad = out.t().reshape(w.shape).to(w.dtype).contiguous()  # [p, d] (conv: [C_out, C_in, kH, kW])
            if bout is not None:
                L.module.bias.grad = bout.to(L.module.bias.dtype)
            L.a = L.g = None
        self.last_norms = norms
        return norms
