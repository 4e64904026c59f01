"""Helpers for the GPU tests: move seeded numpy inputs to the device, call the
HIP library through its C ABI (the Python binding), and bring results back.
Every output buffer they hand to the library sits between 4 KiB guard zones
that are checked after the call."""
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


GUARD = 4096    # bytes of guard zone on each side of every output buffer
PATTERN = 0xA5  # the guard bytes


class Guarded:
    """Output buffers with 4 KiB guard zones before and after them.  Each
    buffer is a view into a larger allocation whose guard bytes hold PATTERN;
    check() asserts that no call wrote outside the buffers it was given."""

    def __init__(self):
        self.bufs = []

    def alloc(self, shape, dtype, fill=None):
        torch = torch_cuda()
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        base = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        t = base[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            t.fill_(fill)
        self.bufs.append((base, n))
        return t

    def check(self):
        for base, n in self.bufs:
            head, tail = base[:GUARD], base[GUARD + n:]
            assert bool((head == PATTERN).all()) and bool((tail == PATTERN).all()), \
                "a kernel wrote outside its output buffer"


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
    g = Guarded()
    u8 = torch.uint8
    if layout == nv.NVFP4_COL_1D:
        codes = g.alloc((cols, rows // 2), u8)
        scales = g.alloc((cols, rows // 16), u8)
    elif layout == nv.NVFP4_ROW_1D:
        codes = g.alloc((rows, cols // 2), u8)
        scales = g.alloc((rows, cols // 16), u8)
    else:
        codes = g.alloc((rows, cols // 2), u8)
        scales = g.alloc((rows // 16, cols // 16), u8)
    codes_t = scales_t = None
    if layout == nv.NVFP4_TILE_2D and transpose:
        codes_t = g.alloc((cols, rows // 2), u8)
        scales_t = g.alloc((cols // 16, rows // 16), u8)
    ts = g.alloc((1,), torch.float32)
    am = g.alloc((1,), torch.float32)
    nv.nvfp4_quantize(xd, dtype_code(x), rows, cols, ld, layout, rnd, seed, codes, scales,
                      codes_t, scales_t, ts, am)
    torch.cuda.synchronize()
    g.check()
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
    g = Guarded()
    codes = g.alloc((cols, tokens // 2), torch.uint8)
    scales = g.alloc((cols, tokens // 16), torch.uint8)
    ts = g.alloc((1,), torch.float32)
    am = g.alloc((1,), torch.float32)
    nv.nvfp4_rht_quantize(xd, dtype_code(x), tokens, cols, cols, sign_mask, rnd, seed, codes,
                          scales, ts, am)
    torch.cuda.synchronize()
    g.check()
    return dict(codes=host(codes), scales=host(scales), tensor_scale=float(host(ts)[0]),
                amax=float(host(am)[0]), dev=dict(codes=codes, scales=scales, ts=ts))


def gpu_quantize_row_rht(x: np.ndarray, sign_mask: int, row_rnd: int, row_seed: int, rht_rnd: int,
                         rht_seed: int, ld: int | None = None, pad=0) -> tuple[dict, dict]:
    """nvfp4_quantize_row_rht: (row-1D outputs, RHT column outputs), both as
    returned by gpu_quantize / gpu_rht_quantize.  With ld > cols the input
    rows are ld elements apart and the gap holds `pad` (which no output may
    depend on)."""
    torch = torch_cuda()
    tokens, cols = x.shape
    if ld is not None and ld != cols:
        padded = np.full((tokens, ld), pad, dtype=x.dtype)
        padded[:, :cols] = x
        xd = to_dev(padded)
    else:
        ld = cols
        xd = to_dev(x)
    g = Guarded()
    u8 = torch.uint8
    rc, rs = g.alloc((tokens, cols // 2), u8), g.alloc((tokens, cols // 16), u8)
    hc, hs = g.alloc((cols, tokens // 2), u8), g.alloc((cols, tokens // 16), u8)
    rts, ram, hts, ham = (g.alloc((1,), torch.float32) for _ in range(4))
    nv.nvfp4_quantize_row_rht(xd, dtype_code(x), tokens, cols, ld, row_rnd, row_seed, rc, rs, rts, ram,
                              sign_mask, rht_rnd, rht_seed, hc, hs, hts, ham)
    torch.cuda.synchronize()
    g.check()
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
    g = Guarded()
    if layout == nv.NVFP4_COL_1D:
        codes = g.alloc((cols, rows // 2), torch.uint8)
        scales = g.alloc((cols, rows // 32), torch.uint8)
    else:
        codes = g.alloc((rows, cols // 2), torch.uint8)
        scales = g.alloc((rows, cols // 32), torch.uint8)
    nv.mxfp4_quantize(xd, dtype_code(x), rows, cols, cols, layout, rnd, seed, codes, scales)
    torch.cuda.synchronize()
    g.check()
    return dict(codes=host(codes), scales=host(scales), dev=dict(codes=codes, scales=scales))


def gpu_mx_gemm(M, N, K, a: dict, b: dict, c0: np.ndarray | None = None, beta: float = 0.0,
                workspace="auto") -> np.ndarray:
    torch = torch_cuda()
    g = Guarded()
    c = g.alloc((M, N), torch.float32, fill=0.0)
    if c0 is not None:
        c.copy_(to_dev(np.ascontiguousarray(c0, dtype=np.float32)))
    if isinstance(workspace, str):
        workspace = nv.nvfp4_gemm_workspace_size(M, N, K)
    ws = g.alloc((workspace // 4,), torch.float32, fill=float("nan")) if workspace else None
    nv.mxfp4_gemm(M, N, K, a["codes"], a["scales"], b["codes"], b["scales"], c, N, beta, workspace=ws)
    torch.cuda.synchronize()
    g.check()
    return host(c)


def gpu_gemm(M, N, K, a: dict, b: dict, b_rowdiv: int, c0: np.ndarray | None = None,
             beta: float = 0.0, workspace="auto") -> np.ndarray:
    """C = beta*C0 + A.B^T from device-resident quantize outputs a, b (dicts with
    dev codes/scales/ts as returned above; b may name its transposed copy).
    workspace: "auto" allocates the size the library asks for, None passes NULL,
    an int passes a workspace of that many bytes."""
    torch = torch_cuda()
    g = Guarded()
    c = g.alloc((M, N), torch.float32, fill=0.0)
    if c0 is not None:
        c.copy_(to_dev(np.ascontiguousarray(c0, dtype=np.float32)))
    if isinstance(workspace, str):
        workspace = nv.nvfp4_gemm_workspace_size(M, N, K)
    ws = None
    if workspace:
        # filled with NaN so that a partial tile the kernel failed to write shows
        ws = g.alloc((workspace // 4,), torch.float32, fill=float("nan"))
    nv.nvfp4_gemm(M, N, K, a["codes"], a["scales"], a["ts"], b["codes"], b["scales"], b_rowdiv,
                  b["ts"], c, N, beta, workspace=ws)
    torch.cuda.synchronize()
    g.check()
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
