"""Helpers for the GPU tests: move seeded numpy inputs to the device, call the
HIP library through its C ABI (the Python binding), and bring results back."""
from __future__ import annotations

import numpy as np

import bit_microscaled_quantized_amd as nv


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dtype_code(a: np.ndarray) -> int:
    return nv.NVFP4_BF16 if a.dtype == np.uint16 else nv.NVFP4_F32


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def gpu_quantize(x: np.ndarray, layout: int, rnd: int = 0, seed: int = 0, ld: int | None = None,
                 transpose: bool = True) -> dict:
    """Quantize x (rows x cols; bf16 bits or fp32) on the GPU.  With ld > cols
    the input is laid out with that leading dimension (padding = NaN-free 0)."""
    torch = torch_cuda()
    rows, cols = x.shape
    if ld is not None and ld != cols:
        pad = np.zeros((rows, ld), dtype=x.dtype)
        pad[:, :cols] = x
        xd = to_dev(pad)
    else:
        ld = cols
        xd = to_dev(x)
    u8 = dict(dtype=torch.uint8, device="cuda")
    if layout == nv.NVFP4_COL_1D:
        codes = torch.empty((cols, rows // 2), **u8)
        scales = torch.empty((cols, rows // 16), **u8)
    elif layout == nv.NVFP4_ROW_1D:
        codes = torch.empty((rows, cols // 2), **u8)
        scales = torch.empty((rows, cols // 16), **u8)
    else:
        codes = torch.empty((rows, cols // 2), **u8)
        scales = torch.empty((rows // 16, cols // 16), **u8)
    codes_t = scales_t = None
    if layout == nv.NVFP4_TILE_2D and transpose:
        codes_t = torch.empty((cols, rows // 2), **u8)
        scales_t = torch.empty((cols // 16, rows // 16), **u8)
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_quantize(xd, dtype_code(x), rows, cols, ld, layout, rnd, seed, codes, scales,
                      codes_t, scales_t, ts, am)
    torch.cuda.synchronize()
    out = dict(codes=host(codes), scales=host(scales), tensor_scale=float(host(ts)[0]),
               amax=float(host(am)[0]), dev=dict(codes=codes, scales=scales, ts=ts,
                                                 codes_t=codes_t, scales_t=scales_t))
    if codes_t is not None:
        out.update(codes_t=host(codes_t), scales_t=host(scales_t))
    return out


def gpu_rht_quantize(x: np.ndarray, sign_mask: int, rnd: int = 0, seed: int = 0) -> dict:
    torch = torch_cuda()
    tokens, cols = x.shape
    xd = to_dev(x)
    codes = torch.empty((cols, tokens // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((cols, tokens // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_rht_quantize(xd, dtype_code(x), tokens, cols, cols, sign_mask, rnd, seed, codes,
                          scales, ts, am)
    torch.cuda.synchronize()
    return dict(codes=host(codes), scales=host(scales), tensor_scale=float(host(ts)[0]),
                amax=float(host(am)[0]), dev=dict(codes=codes, scales=scales, ts=ts))


def gpu_quantize_row_rht(x: np.ndarray, sign_mask: int, row_rnd: int, row_seed: int, rht_rnd: int,
                         rht_seed: int) -> tuple[dict, dict]:
    """nvfp4_quantize_row_rht: (row-1D outputs, RHT column outputs), both as
    returned by gpu_quantize / gpu_rht_quantize."""
    torch = torch_cuda()
    tokens, cols = x.shape
    xd = to_dev(x)
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    rc, rs = torch.empty((tokens, cols // 2), **u8), torch.empty((tokens, cols // 16), **u8)
    hc, hs = torch.empty((cols, tokens // 2), **u8), torch.empty((cols, tokens // 16), **u8)
    rts, ram, hts, ham = (torch.empty(1, **f32) for _ in range(4))
    nv.nvfp4_quantize_row_rht(xd, dtype_code(x), tokens, cols, cols, row_rnd, row_seed, rc, rs, rts, ram,
                              sign_mask, rht_rnd, rht_seed, hc, hs, hts, ham)
    torch.cuda.synchronize()
    row = dict(codes=host(rc), scales=host(rs), tensor_scale=float(host(rts)[0]), amax=float(host(ram)[0]),
               dev=dict(codes=rc, scales=rs, ts=rts))
    rht = dict(codes=host(hc), scales=host(hs), tensor_scale=float(host(hts)[0]), amax=float(host(ham)[0]),
               dev=dict(codes=hc, scales=hs, ts=hts))
    return row, rht


def gpu_mx_quantize(x: np.ndarray, layout: int, rnd: int = 0, seed: int = 0) -> dict:
    """mxfp4_quantize of x (rows x cols; bf16 bits or fp32) on the GPU."""
    torch = torch_cuda()
    rows, cols = x.shape
    xd = to_dev(x)
    u8 = dict(dtype=torch.uint8, device="cuda")
    if layout == nv.NVFP4_COL_1D:
        codes = torch.empty((cols, rows // 2), **u8)
        scales = torch.empty((cols, rows // 32), **u8)
    else:
        codes = torch.empty((rows, cols // 2), **u8)
        scales = torch.empty((rows, cols // 32), **u8)
    nv.mxfp4_quantize(xd, dtype_code(x), rows, cols, cols, layout, rnd, seed, codes, scales)
    torch.cuda.synchronize()
    return dict(codes=host(codes), scales=host(scales), dev=dict(codes=codes, scales=scales))


def gpu_mx_gemm(M, N, K, a: dict, b: dict, c0: np.ndarray | None = None, beta: float = 0.0,
                workspace="auto") -> np.ndarray:
    torch = torch_cuda()
    c = torch.zeros((M, N), dtype=torch.float32, device="cuda") if c0 is None else \
        to_dev(np.ascontiguousarray(c0, dtype=np.float32))
    if isinstance(workspace, str):
        workspace = nv.nvfp4_gemm_workspace_size(M, N, K)
    ws = torch.full((workspace // 4,), float("nan"), dtype=torch.float32, device="cuda") if workspace else None
    nv.mxfp4_gemm(M, N, K, a["codes"], a["scales"], b["codes"], b["scales"], c, N, beta, workspace=ws)
    torch.cuda.synchronize()
    return host(c)


def gpu_gemm(M, N, K, a: dict, b: dict, b_rowdiv: int, c0: np.ndarray | None = None,
             beta: float = 0.0, workspace="auto") -> np.ndarray:
    """C = beta*C0 + A.B^T from device-resident quantize outputs a, b (dicts with
    dev codes/scales/ts as returned above; b may name its transposed copy).
    workspace: "auto" allocates the size the library asks for, None passes NULL,
    an int passes a workspace of that many bytes."""
    torch = torch_cuda()
    if c0 is None:
        c = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    else:
        c = to_dev(np.ascontiguousarray(c0, dtype=np.float32))
    if isinstance(workspace, str):
        workspace = nv.nvfp4_gemm_workspace_size(M, N, K)
    ws = None
    if workspace:
        # filled with NaN so that a partial tile the kernel failed to write shows
        ws = torch.full((workspace // 4,), float("nan"), dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm(M, N, K, a["codes"], a["scales"], a["ts"], b["codes"], b["scales"], b_rowdiv,
                  b["ts"], c, N, beta, workspace=ws)
    torch.cuda.synchronize()
    return host(c)


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return "identical"
    i = tuple(idx[0])
    return f"{len(idx)} differing entries; first at {i}: gpu={a[i]} oracle={b[i]}"


def rel_fro(c: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(c, np.float64) - ref) / np.linalg.norm(ref))
