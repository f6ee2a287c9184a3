"""Training-step integration of the INSTANT low-rank backward: a bias-free linear layer
y = x w^T whose backward runs through the library (notes "INSTANT: Compressing Gradients
and Activations for Resource-Efficient Training", 整体框架: calibrate every N_t steps,
compress and run the low-rank backward in between; 关键设计 3 for the backward).

Schedule of each window of N_t training steps (the library leaves it to the caller):

  - steps 0 .. N_cal-1 of the window are calibration steps: the forward keeps x, the
    backward is exact (PyTorch GEMMs) and also hands x and g_y to the library's
    statistics; the last of them finalizes, which installs the new P and Q;
  - the other steps keep only x_hat = P x from the forward (the activation memory saving)
    and run the library's low-rank backward.

Until a finalize has succeeded there are no projections, and a step that is not a
calibration step falls back to the exact backward. A failed finalize keeps the previous
projections (the library's rule), so the layer keeps compressing with them.

Only the forward GEMM and the exact backward of calibration steps are PyTorch's; every
step of the INSTANT path (statistics, decomposition, truncation, compression, low-rank
backward) runs in the HIP kernels of libinstant.so. One forward and one backward per step,
in order, on the layer's device.
"""
from __future__ import annotations

import math

import torch

from . import INSTANT_OK, InstantLayer, instant_status_str, make_config


class _InstantLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, mod, mode):
        y = torch.nn.functional.linear(x, w)  # the caller's GEMM
        B = x.shape[0]
        if mode == "compress":
            xhat = torch.empty((B, mod.Rx, mod.Cx), dtype=x.dtype, device=x.device)
            mod.layer.compress_fwd(x, B, xhat)
            ctx.save_for_backward(xhat, w)
        else:
            ctx.save_for_backward(x, w)
        ctx.mod, ctx.mode = mod, mode
        return y

    @staticmethod
    def backward(ctx, gy):
        saved, w = ctx.saved_tensors
        mod, mode = ctx.mod, ctx.mode
        gy = gy.contiguous()
        B = gy.shape[0]
        if mode == "compress":
            gw = torch.empty_like(w)
            gx = torch.empty((B, mod.L, mod.Cx), dtype=gy.dtype, device=gy.device)
            mod.layer.backward(saved, gy, w, B, gw, gx)
            return gx, gw, None, None
        x = saved
        gx = torch.matmul(gy.reshape(-1, mod.Cy), w).reshape(B, mod.L, mod.Cx)
        gw = torch.mm(gy.reshape(-1, mod.Cy).t().contiguous(), x.reshape(-1, mod.Cx))
        if mode in ("calibrate", "finalize"):
            mod._calibrate(x, gy, B, finalize=(mode == "finalize"))
        return gx, gw, None, None


class InstantLinear(torch.nn.Module):
    """y = x w^T for x [B, L, Cx] -> y [B, L, Cy], weight [Cy, Cx], with the INSTANT
    backward on the steps between calibrations.

    dtype is the library's I/O dtype ("bf16" or "fp32"); inputs and the weight must have
    it. N_cal calibration steps start every window of N_t steps (N_cal <= N_t).

    comp is the energy compensation of the projections (关键设计 2). The default is the
    ratio reading, c = (E / sum_{i<=R} sigma_i^2)^(1/2) >= 1, which keeps the compressed
    steps' gradients on the scale of the exact ones. The factor as printed ("paper",
    c = (sum_{i<=R} sigma_i^2)^(-1/2)) carries the units of the data: g_w scales by c_P^2
    and g_x by c_Q^2 (about 5e-11 on BERT-sized synthetic data), so the compressed steps of a
    window would get gradients on a different scale from its exact calibration steps; it
    stays selectable. "none" (c = 1) gives the orthogonal projection.
    """

    def __init__(self, L, Cx, Cy, B_max, N_t=100, N_cal=16, p=2, eps=0.95, dtype="bf16", R_max=64,
                 comp="ratio", weight=None, device="cuda"):
        super().__init__()
        if not 1 <= N_cal <= N_t:
            raise ValueError("need 1 <= N_cal <= N_t")
        self.L, self.Cx, self.Cy, self.B_max = int(L), int(Cx), int(Cy), int(B_max)
        self.N_t, self.N_cal = int(N_t), int(N_cal)
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        if weight is None:
            weight = torch.randn(Cy, Cx, device=device) / math.sqrt(Cx)
        self.weight = torch.nn.Parameter(weight.to(device=device, dtype=self.torch_dtype).contiguous())
        self.layer = InstantLayer(make_config(L, Cx, Cy, B_max, R_max=R_max, p=p, N_t=N_t, eps=eps,
                                              dtype=dtype, comp=comp), device=device)
        self.step = 0          # training steps whose forward has run
        self.generation = 0    # successful finalizes so far
        self.Rx = self.Ry = 0
        self.last_status = INSTANT_OK

    def mode_of_step(self, step: int) -> str:
        t = step % self.N_t
        if t < self.N_cal:
            return "finalize" if t == self.N_cal - 1 else "calibrate"
        return "compress" if self.generation > 0 else "exact"

    def _calibrate(self, x, gy, B, finalize):
        s = self.layer.calibrate(x, gy, B, finalize=finalize)
        if finalize:
            self.last_status = s
            if s == INSTANT_OK:
                _, info = self.layer.query()
                self.generation += 1
                self.Rx, self.Ry = info.Rx, info.Ry

    def forward(self, x):
        if x.dim() != 3 or x.shape[1] != self.L or x.shape[2] != self.Cx or x.shape[0] > self.B_max:
            raise ValueError(f"x must be [B <= {self.B_max}, {self.L}, {self.Cx}], got {tuple(x.shape)}")
        if x.dtype != self.torch_dtype:
            raise TypeError(f"x must be {self.torch_dtype}")
        x = x.contiguous()
        if not (self.training and torch.is_grad_enabled()):
            return torch.nn.functional.linear(x, self.weight)
        mode = self.mode_of_step(self.step)
        self.step += 1
        return _InstantLinearFn.apply(x, self.weight, self, mode)

    def status(self) -> str:
        return instant_status_str(self.last_status)
