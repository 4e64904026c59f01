"""NVFP4 linear layer for PyTorch autograd, on the libnvfp4 kernels.

The recipe ("Pretraining Large Language Models with NVFP4", gist.science
summary, Resumo tecnico, 2. Metodologia Proposta) applied per GEMM:

  forward   Y  = X W^T : X row-1D RNE, W 16x16 2D RNE                (technique 3)
  backward  dX = dY W  : dY row-1D SR, the same 2D-quantized W, transposed
            dW = dY^T X: dY and X through the 16x16 random Hadamard transform
                         along tokens (one sign mask per layer), column-1D;
                         SR on dY, RNE on X                        (techniques 2, 4)

Technique 1 of the same part keeps a minority of layers in BF16: a layer
built with `bf16=True` runs the plain BF16 product instead (torch's matmul),
with no quantization at all.

Forward quantizes W and X (X's row copy for Fprop and its RHT column copy for
Wgrad, from one read) and keeps only the quantized operands for backward: the
saved activations are 4.5 bits per element.  Outputs and gradients come back in
the dtype of the corresponding input (BF16 through nvfp4_gemm_bf16, FP32
through nvfp4_gemm).  Every quantize, GEMM and rounding step runs in libnvfp4
on torch's current stream; this module only allocates the buffers and orders
the calls.  The buffers come from PyTorch's caching allocator, so from the
second step on they are blocks it already holds and a step makes no device
allocation call.  W is quantized once per forward (the weights change with
every optimizer step); backward reuses that call's transposed copy.

Shapes: x [..., in_features] with the flattened token count a multiple of 64,
in_features and out_features multiples of 64 (each is the K of one GEMM).
Stochastic rounding draws its bits from the counter-based hash keyed by a
per-call seed: seed_base + 2 * call (row copy of dY) and + 1 (RHT copy), so a
layer built with the same seed reproduces its gradients bit for bit.
"""
from __future__ import annotations

import numpy as np

from . import nvfp4 as nv

_DT = {}


def _dt(torch, t) -> int:
    if not _DT:
        _DT[torch.bfloat16] = nv.NVFP4_BF16
        _DT[torch.float32] = nv.NVFP4_F32
    if t.dtype not in _DT:
        raise TypeError(f"NVFP4Linear takes bfloat16 or float32 tensors, got {t.dtype}")
    return _DT[t.dtype]


def _quantized(torch, rows, cols, dev, tiles=False):
    """Buffers of one quantized copy: codes [rows][cols/2], scales (1D or 16x16
    tiles), tensor scale and amax."""
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    srows = rows // 16 if tiles else rows
    return dict(codes=torch.empty((rows, cols // 2), **u8),
                scales=torch.empty((srows, cols // 16), **u8),
                ts=torch.empty(1, **f32), amax=torch.empty(1, **f32))


def _gemm(torch, M, N, K, a, b, b_rowdiv, out_dtype, dev, b_codes="codes", b_scales="scales"):
    """C[M][N] = A . B^T of two quantized operands, in out_dtype."""
    c = torch.empty((M, N), dtype=out_dtype, device=dev)
    ws_bytes = nv.nvfp4_gemm_workspace_size(M, N, K)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    fn = nv.nvfp4_gemm_bf16 if out_dtype == torch.bfloat16 else nv.nvfp4_gemm
    fn(M, N, K, a["codes"], a["scales"], a["ts"], b[b_codes], b[b_scales], b_rowdiv, b["ts"], c, N,
       0.0, workspace=ws)
    return c


def _function():
    import torch

    class NVFP4LinearFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w, sign_mask: int, seed_row: int, seed_col: int):
            dev = x.device
            IN = x.shape[-1]
            OUT = w.shape[0]
            x2 = x.reshape(-1, IN).contiguous()
            wc = w.contiguous()
            T = x2.shape[0]
            for name, v in (("tokens", T), ("in_features", IN), ("out_features", OUT)):
                if v <= 0 or v % 64 != 0:
                    raise ValueError(f"NVFP4Linear needs {name} a positive multiple of 64, got {v}")
            qw = _quantized(torch, OUT, IN, dev, tiles=True)
            qw["codes_t"] = torch.empty((IN, OUT // 2), dtype=torch.uint8, device=dev)
            qw["scales_t"] = torch.empty((IN // 16, OUT // 16), dtype=torch.uint8, device=dev)
            nv.nvfp4_quantize(wc, _dt(torch, wc), OUT, IN, IN, nv.NVFP4_TILE_2D, nv.NVFP4_RNE, 0,
                              qw["codes"], qw["scales"], qw["codes_t"], qw["scales_t"], qw["ts"],
                              qw["amax"])
            qx = _quantized(torch, T, IN, dev)
            qxt = _quantized(torch, IN, T, dev)
            nv.nvfp4_quantize_row_rht(x2, _dt(torch, x2), T, IN, IN, nv.NVFP4_RNE, 0, qx["codes"],
                                      qx["scales"], qx["ts"], qx["amax"], sign_mask, nv.NVFP4_RNE,
                                      0, qxt["codes"], qxt["scales"], qxt["ts"], qxt["amax"])
            y = _gemm(torch, T, OUT, IN, qx, qw, 16, x.dtype, dev)
            ctx.save_for_backward(qw["codes_t"], qw["scales_t"], qw["ts"], qxt["codes"],
                                  qxt["scales"], qxt["ts"])
            ctx.meta = (T, IN, OUT, sign_mask, seed_row, seed_col, x.shape, x.dtype, w.dtype)
            return y.reshape(*x.shape[:-1], OUT)

        @staticmethod
        def backward(ctx, dy):
            wct, wst, wts, xc, xs, xts = ctx.saved_tensors
            T, IN, OUT, sign_mask, seed_row, seed_col, x_shape, x_dtype, w_dtype = ctx.meta
            dev = dy.device
            dy2 = dy.reshape(T, OUT).contiguous()
            qd = _quantized(torch, T, OUT, dev)
            qdt = _quantized(torch, OUT, T, dev)
            nv.nvfp4_quantize_row_rht(dy2, _dt(torch, dy2), T, OUT, OUT, nv.NVFP4_SR, seed_row,
                                      qd["codes"], qd["scales"], qd["ts"], qd["amax"], sign_mask,
                                      nv.NVFP4_SR, seed_col, qdt["codes"], qdt["scales"],
                                      qdt["ts"], qdt["amax"])
            qw = dict(codes=wct, scales=wst, ts=wts)
            qxt = dict(codes=xc, scales=xs, ts=xts)
            dx = _gemm(torch, T, IN, OUT, qd, qw, 16, x_dtype, dev)
            dw = _gemm(torch, OUT, IN, T, qdt, qxt, 1, w_dtype, dev)
            return dx.reshape(x_shape), dw, None, None, None

    return NVFP4LinearFn


_FN = None


def nvfp4_linear(x, w, sign_mask: int, seed_row: int, seed_col: int):
    """y = x w^T with NVFP4 GEMMs in forward and backward (autograd-aware)."""
    global _FN
    if _FN is None:
        _FN = _function()
    return _FN.apply(x, w, int(sign_mask) & 0xFFFF, int(seed_row), int(seed_col))


def _module_base():
    import torch
    return torch.nn.Module


class NVFP4Linear(_module_base()):
    """Bias-free linear layer whose Fprop, Dgrad and Wgrad run on NVFP4
    operands (or, with bf16=True, a plain BF16 layer)."""

    def __init__(self, in_features: int, out_features: int, bf16: bool = False, seed: int = 0,
                 device="cuda", dtype=None):
        import torch
        super().__init__()
        self.in_features, self.out_features, self.bf16 = in_features, out_features, bf16
        dtype = dtype or torch.bfloat16
        w = torch.empty((out_features, in_features), dtype=torch.float32)
        torch.nn.init.normal_(w, 0.0, in_features ** -0.5, generator=torch.Generator().manual_seed(seed))
        self.weight = torch.nn.Parameter(w.to(device=device, dtype=dtype))
        rng = np.random.default_rng(seed)
        self.sign_mask = int(rng.integers(0, 1 << 16))
        self.seed_base = int(rng.integers(0, 1 << 62))
        self.calls = 0

    def forward(self, x):
        import torch
        if self.bf16:
            return torch.nn.functional.linear(x, self.weight)
        s = self.seed_base + 2 * self.calls
        self.calls += 1
        return nvfp4_linear(x, self.weight, self.sign_mask, s, s + 1)
