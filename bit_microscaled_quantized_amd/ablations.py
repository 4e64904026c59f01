"""Measurement-only ablations of two choices of the recipe, run on the GPU
quantize and dequantize kernels.

"Pretraining Large Language Models with NVFP4" (gist.science summary),
Resumo tecnico, 2. Metodologia Proposta:

* technique 3 (2D weight scaling): with 1D scales along the contraction
  dimension, Fprop's weight (blocks along W's rows) and Dgrad's weight (blocks
  along W's columns) are two different quantizations of W, so the backward pass
  differentiates a different function than the forward pass computed; 16x16
  tiles make the two one and the same.
* technique 2 (random Hadamard transform on the Wgrad inputs): mixing each
  16-token block spreads its outliers, lowering the block's crest factor
  (max |y| / rms y), so less of the E2M1 range is wasted on a few values.

weight_consistency(w) quantizes W with 1D row scales, 1D column scales and 2D
tiles (with the transposed copy), dequantizes every copy to FP32 on the GPU
and reports
  mismatch_1d = ||deq(row) - deq(col)^T||_F / ||W||_F   (> 0)
  mismatch_2d = ||deq(2D) - deq(2D^T)^T||_F / ||W||_F   (exactly 0)
  error_1d_row, error_1d_col, error_2d = ||deq - W||_F / ||W||_F.
rht_effect(x, sign_mask) quantizes x column-1D along tokens (the Wgrad
layout) without and with the transform and reports
  crest_plain, crest_rht: mean over 16-token blocks of max|y| / rms(y)
  error_plain, error_rht: ||deq - y||_F / ||y||_F, y = x or RHT(x).
The transform is orthonormal, so error_rht is also the error of the
back-transformed values.  Element-wise error is not what the transform is for:
wgrad_effect(dy, x, sign_mask) measures the quantity it serves, the Wgrad
product, quantized as the recipe does it (dY with SR, X with RNE, both
column-1D along tokens) without and with the shared transform:
  wgrad_error_plain, wgrad_error_rht = ||C - dY^T X||_F / ||dY^T X||_F
with C the NVFP4 GEMM of the two quantized copies (the transform cancels in
the product, so C estimates dY^T X in both cases).  The statistics (norms, the reference transform of x
for error_rht) are measurement, computed with torch in FP64 from the kernels'
outputs; nothing here is part of the quantize-and-contract path.

    python -m bit_microscaled_quantized_amd.ablations   # full-size run, one JSON line
"""
from __future__ import annotations

import json

import numpy as np

from . import nvfp4 as nv


def _torch():
    import torch
    return torch


def _dev_bf16(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _quant(torch, x, rows, cols, layout):
    """nvfp4_quantize of a bf16 device tensor; returns the stored codes,
    scales (and transposed copy for 2D) and the tensor scale."""
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    if layout == nv.NVFP4_COL_1D:
        codes, scales = torch.empty((cols, rows // 2), **u8), torch.empty((cols, rows // 16), **u8)
        ct = st = None
    elif layout == nv.NVFP4_ROW_1D:
        codes, scales = torch.empty((rows, cols // 2), **u8), torch.empty((rows, cols // 16), **u8)
        ct = st = None
    else:
        codes, scales = torch.empty((rows, cols // 2), **u8), torch.empty((rows // 16, cols // 16), **u8)
        ct, st = torch.empty((cols, rows // 2), **u8), torch.empty((cols // 16, rows // 16), **u8)
    ts, am = torch.empty(1, **f32), torch.empty(1, **f32)
    nv.nvfp4_quantize(x, nv.NVFP4_BF16, rows, cols, cols, layout, nv.NVFP4_RNE, 0, codes, scales, ct, st,
                      ts, am)
    return dict(codes=codes, scales=scales, codes_t=ct, scales_t=st, ts=ts)


def _deq(torch, codes, scales, rowdiv, ts):
    """FP32 dequantization of stored codes on the GPU (nvfp4_dequantize)."""
    rows, cols = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    nv.nvfp4_dequantize(codes, scales, rowdiv, ts, rows, cols, nv.NVFP4_F32, out, cols)
    return out


def _rel(torch, a, b, ref_norm) -> float:
    return float(torch.linalg.vector_norm((a.double() - b.double()).reshape(-1)) / ref_norm)


def weight_consistency(w_bits: np.ndarray) -> dict:
    """w_bits: bf16 bit patterns of W [out][in]."""
    torch = _torch()
    O, I = w_bits.shape
    w = _dev_bf16(torch, w_bits)
    wf = w.float()
    nrm = float(torch.linalg.vector_norm(wf.double().reshape(-1)))
    r = _quant(torch, w, O, I, nv.NVFP4_ROW_1D)
    c = _quant(torch, w, O, I, nv.NVFP4_COL_1D)
    t = _quant(torch, w, O, I, nv.NVFP4_TILE_2D)
    d_row = _deq(torch, r["codes"], r["scales"], 1, r["ts"])
    d_col = _deq(torch, c["codes"], c["scales"], 1, c["ts"]).t()
    d_2d = _deq(torch, t["codes"], t["scales"], 16, t["ts"])
    d_2dt = _deq(torch, t["codes_t"], t["scales_t"], 16, t["ts"]).t()
    out = dict(mismatch_1d=_rel(torch, d_row, d_col, nrm), mismatch_2d=_rel(torch, d_2d, d_2dt, nrm),
               error_1d_row=_rel(torch, d_row, wf, nrm), error_1d_col=_rel(torch, d_col, wf, nrm),
               error_2d=_rel(torch, d_2d, wf, nrm))
    torch.cuda.synchronize()
    return out


def _rht_f64(torch, y, sign_mask: int):
    """(1/4) H16 diag(d) applied to consecutive 16-token groups of each row of
    y [C][T] (FP64), the transform the RHT quantizer applies before scaling."""
    h = np.array([[(-1.0) ** bin(j & k).count("1") for k in range(16)] for j in range(16)])
    d = np.array([-1.0 if (sign_mask >> j) & 1 else 1.0 for j in range(16)])
    m = torch.from_numpy(0.25 * h * d[None, :]).to(y.device)  # y_j = sum_k m[j][k] x_k
    C, T = y.shape
    return (y.reshape(C, T // 16, 16) @ m.t().contiguous()).reshape(C, T)


def _crest(torch, y) -> float:
    b = y.reshape(-1, 16)
    mx = b.abs().amax(dim=1)
    rms = b.pow(2).mean(dim=1).sqrt()
    keep = rms > 0
    return float((mx[keep] / rms[keep]).mean())


def rht_effect(x_bits: np.ndarray, sign_mask: int) -> dict:
    """x_bits: bf16 bit patterns of a Wgrad operand [tokens][cols]."""
    torch = _torch()
    T, C = x_bits.shape
    x = _dev_bf16(torch, x_bits)
    y_plain = x.double().t().contiguous()  # [C][T], the column-1D layout
    y_rht = _rht_f64(torch, y_plain, sign_mask)
    p = _quant(torch, x, T, C, nv.NVFP4_COL_1D)
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    rc, rs = torch.empty((C, T // 2), **u8), torch.empty((C, T // 16), **u8)
    rts, ram = torch.empty(1, **f32), torch.empty(1, **f32)
    nv.nvfp4_rht_quantize(x, nv.NVFP4_BF16, T, C, C, sign_mask, nv.NVFP4_RNE, 0, rc, rs, rts, ram)
    d_plain = _deq(torch, p["codes"], p["scales"], 1, p["ts"])
    d_rht = _deq(torch, rc, rs, 1, rts)
    n_plain = float(torch.linalg.vector_norm(y_plain.reshape(-1)))
    n_rht = float(torch.linalg.vector_norm(y_rht.reshape(-1)))
    out = dict(crest_plain=_crest(torch, y_plain), crest_rht=_crest(torch, y_rht),
               error_plain=_rel(torch, d_plain, y_plain, n_plain), error_rht=_rel(torch, d_rht, y_rht, n_rht))
    torch.cuda.synchronize()
    return out


def _qcol(torch, t, T, C, rht: bool, sign_mask: int, rnd: int, seed: int):
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    q = dict(codes=torch.empty((C, T // 2), **u8), scales=torch.empty((C, T // 16), **u8),
             ts=torch.empty(1, **f32), amax=torch.empty(1, **f32))
    if rht:
        nv.nvfp4_rht_quantize(t, nv.NVFP4_BF16, T, C, C, sign_mask, rnd, seed, q["codes"], q["scales"],
                              q["ts"], q["amax"])
    else:
        nv.nvfp4_quantize(t, nv.NVFP4_BF16, T, C, C, nv.NVFP4_COL_1D, rnd, seed, q["codes"], q["scales"],
                          None, None, q["ts"], q["amax"])
    return q


def wgrad_effect(dy_bits: np.ndarray, x_bits: np.ndarray, sign_mask: int, seed: int = 1) -> dict:
    """dy_bits [tokens][out], x_bits [tokens][in]: bf16 bit patterns."""
    torch = _torch()
    T, O = dy_bits.shape
    I = x_bits.shape[1]
    dy, x = _dev_bf16(torch, dy_bits), _dev_bf16(torch, x_bits)
    exact = dy.double().t().contiguous() @ x.double()  # [O][I]
    nrm = float(torch.linalg.vector_norm(exact.reshape(-1)))
    out = {}
    for name, rht in (("plain", False), ("rht", True)):
        a = _qcol(torch, dy, T, O, rht, sign_mask, nv.NVFP4_SR, seed)
        b = _qcol(torch, x, T, I, rht, sign_mask, nv.NVFP4_RNE, 0)
        c = torch.empty((O, I), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(nv.nvfp4_gemm_workspace_size(O, I, T), 16), dtype=torch.uint8, device="cuda")
        nv.nvfp4_gemm(O, I, T, a["codes"], a["scales"], a["ts"], b["codes"], b["scales"], 1, b["ts"], c, I,
                      0.0, workspace=ws)
        out[f"wgrad_error_{name}"] = _rel(torch, c, exact, nrm)
    torch.cuda.synchronize()
    return out


def main():
    from . import synth
    d = synth.ffn_up()
    res = dict(weight_20480x5120_normal=weight_consistency(synth.f32_to_bf16_bits(d["w"])))
    del d
    mask = synth.sign_mask16(7)
    for name, gen in (("8192x5120_student_t3", synth.student_t), ("8192x5120_lognormal", synth.lognormal_signed),
                      ("8192x5120_normal", synth.normal), ("8192x5120_token_outliers", synth.token_outliers)):
        x = synth.f32_to_bf16_bits(gen(6, (8192, 5120)))
        dy = synth.f32_to_bf16_bits(gen(5, (8192, 5120)))
        res[f"x_{name}"] = rht_effect(x, mask)
        res[f"wgrad_{name}"] = wgrad_effect(dy, x, mask, seed=8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
