"""One linear layer's NVFP4 quantize-and-contract step on the GPU.

The recipe ("Pretraining Large Language Models with NVFP4", gist.science
summary, Resumo tecnico, 2. Metodologia Proposta):
  Fprop  Y  = X W^T : X row-1D RNE, W 16x16 2D RNE                (technique 3)
  Dgrad  dX = dY W  : dY row-1D SR, the SAME 2D-quantized W, transposed
  Wgrad  dW = dY^T X: dY and X through the 16x16 random Hadamard transform
                      along tokens (one sign vector for both), column-1D;
                      SR on dY, RNE on X                          (techniques 2, 4)
Shapes: X [T x IN], W [OUT x IN], dY [T x OUT]; Y [T x OUT], dX [T x IN],
dW [OUT x IN].  X and dY each need a row quantization and an RHT column one;
both come from one nvfp4_quantize_row_rht call (one read of the tensor for
the two amaxes): X's in forward (its Wgrad operand is kept for backward), dY's
in backward.  Every step is one call into libnvfp4; this module only owns the
device buffers (allocated once, including the GEMM workspace shared by the three
GEMMs, which therefore must stay on one stream) and the call order.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import nvfp4 as nv


@dataclass
class Quantized:
    codes: object
    scales: object
    ts: object
    amax: object
    codes_t: object = None
    scales_t: object = None


def _alloc_q(torch, rows_out, bytes_per_row, scale_rows, scale_cols, dev, t_shape=None):
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    q = Quantized(torch.empty((rows_out, bytes_per_row), **u8),
                  torch.empty((scale_rows, scale_cols), **u8),
                  torch.empty(1, **f32), torch.empty(1, **f32))
    if t_shape is not None:
        (cr, cb), (sr, sc) = t_shape
        q.codes_t = torch.empty((cr, cb), **u8)
        q.scales_t = torch.empty((sr, sc), **u8)
    return q


class LinearStep:
    """Buffers and call sequence for one layer of shape (tokens, d_in, d_out)."""

    def __init__(self, tokens: int, d_in: int, d_out: int, device="cuda"):
        import torch
        self.torch = torch
        self.T, self.IN, self.OUT = tokens, d_in, d_out
        T, IN, OUT = tokens, d_in, d_out
        self.qx = _alloc_q(torch, T, IN // 2, T, IN // 16, device)
        self.qw = _alloc_q(torch, OUT, IN // 2, OUT // 16, IN // 16, device,
                           t_shape=((IN, OUT // 2), (IN // 16, OUT // 16)))
        self.qdy = _alloc_q(torch, T, OUT // 2, T, OUT // 16, device)
        self.qdy_t = _alloc_q(torch, OUT, T // 2, OUT, T // 16, device)
        self.qx_t = _alloc_q(torch, IN, T // 2, IN, T // 16, device)
        f32 = dict(dtype=torch.float32, device=device)
        self.y = torch.empty((T, OUT), **f32)
        self.dx = torch.empty((T, IN), **f32)
        self.dw = torch.zeros((OUT, IN), **f32)
        ws = max(nv.nvfp4_gemm_workspace_size(T, OUT, IN), nv.nvfp4_gemm_workspace_size(T, IN, OUT),
                 nv.nvfp4_gemm_workspace_size(OUT, IN, T))
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)

    def quantize_weight(self, w, dt, stream=None):
        q = self.qw
        nv.nvfp4_quantize(w, dt, self.OUT, self.IN, self.IN, nv.NVFP4_TILE_2D, nv.NVFP4_RNE, 0,
                          q.codes, q.scales, q.codes_t, q.scales_t, q.ts, q.amax, stream)

    def forward(self, x, dt, sign_mask: int | None = None, stream=None):
        """Y = X W^T.  With the RHT sign mask, X's Wgrad operand is quantized in
        the same call and kept for backward."""
        q = self.qx
        if sign_mask is None:
            nv.nvfp4_quantize(x, dt, self.T, self.IN, self.IN, nv.NVFP4_ROW_1D, nv.NVFP4_RNE, 0,
                              q.codes, q.scales, None, None, q.ts, q.amax, stream)
            self._xt_mask = None
        else:
            b = self.qx_t
            nv.nvfp4_quantize_row_rht(x, dt, self.T, self.IN, self.IN, nv.NVFP4_RNE, 0, q.codes,
                                      q.scales, q.ts, q.amax, sign_mask, nv.NVFP4_RNE, 0, b.codes,
                                      b.scales, b.ts, b.amax, stream)
            self._xt_mask = sign_mask & 0xFFFF
        w = self.qw
        nv.nvfp4_gemm(self.T, self.OUT, self.IN, q.codes, q.scales, q.ts, w.codes, w.scales, 16,
                      w.ts, self.y, self.OUT, 0.0, workspace=self.ws, stream=stream)

    def backward(self, x, dy, dt, sign_mask: int, seed_row: int, seed_col: int,
                 accumulate_wgrad: bool = False, stream=None):
        T, IN, OUT = self.T, self.IN, self.OUT
        q, a, b = self.qdy, self.qdy_t, self.qx_t
        nv.nvfp4_quantize_row_rht(dy, dt, T, OUT, OUT, nv.NVFP4_SR, seed_row, q.codes, q.scales,
                                  q.ts, q.amax, sign_mask, nv.NVFP4_SR, seed_col, a.codes,
                                  a.scales, a.ts, a.amax, stream)
        w = self.qw
        nv.nvfp4_gemm(T, IN, OUT, q.codes, q.scales, q.ts, w.codes_t, w.scales_t, 16, w.ts,
                      self.dx, IN, 0.0, workspace=self.ws, stream=stream)
        if getattr(self, "_xt_mask", None) != (sign_mask & 0xFFFF):
            nv.nvfp4_rht_quantize(x, dt, T, IN, IN, sign_mask, nv.NVFP4_RNE, 0, b.codes, b.scales,
                                  b.ts, b.amax, stream)
        nv.nvfp4_gemm(OUT, IN, T, a.codes, a.scales, a.ts, b.codes, b.scales, 1, b.ts, self.dw,
                      IN, 1.0 if accumulate_wgrad else 0.0, workspace=self.ws, stream=stream)

    def step(self, x, w, dy, dt, sign_mask: int, seed_row: int, seed_col: int,
             accumulate_wgrad: bool = False, quantize_weight: bool = True, stream=None):
        if quantize_weight:
            self.quantize_weight(w, dt, stream)
        self.forward(x, dt, sign_mask, stream)
        self.backward(x, dy, dt, sign_mask, seed_row, seed_col, accumulate_wgrad, stream)
