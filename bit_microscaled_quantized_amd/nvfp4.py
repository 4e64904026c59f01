"""Python binding of libnvfp4 (include/nvfp4.h): argument marshalling only.

Each function has the name and the argument order of its C entry point.  Tensor
arguments may be torch tensors (their data_ptr is passed), raw integer device
addresses, or None for NULL.  `stream=None` means torch's current stream on the
current device.  Every step of the computation runs in the HIP library; if the
library is missing or fails to load, the call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK, NVFP4_EINVAL, NVFP4_ESHAPE, NVFP4_EALIGN, NVFP4_EHIP, NVFP4_ESCRATCH = range(6)
NVFP4_BF16, NVFP4_F32 = 0, 1
NVFP4_RNE, NVFP4_SR = 0, 1
NVFP4_ROW_1D, NVFP4_COL_1D, NVFP4_TILE_2D = 0, 1, 2

EXPORTED = ("nvfp4_quantize", "nvfp4_rht_quantize", "nvfp4_quantize_row_rht", "nvfp4_gemm",
            "nvfp4_gemm_noalloc", "nvfp4_gemm_bf16", "nvfp4_dequantize", "nvfp4_gemm_workspace_size",
            "nvfp4_set_quantize_passes", "nvfp4_set_sync_spin_limit", "nvfp4_single_pass_stats",
            "nvfp4_status_str", "mxfp4_quantize", "mxfp4_gemm")

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libnvfp4.so (built by bit_microscaled_quantized_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m bit_microscaled_quantized_amd.build`")
    # torch first: it ships its own HIP runtime under the same soname, and the
    # library must bind to that one instance (the tensors and streams it is
    # given belong to it); loaded first, the library would pull in the system
    # runtime and torch would then find no usable GPU.
    import torch  # noqa: F401
    L = ctypes.CDLL(_LIB_PATH)
    i64, u64, u32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
    vp, f32 = ctypes.c_void_p, ctypes.c_float
    L.nvfp4_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, u64, vp, vp, vp, vp, vp, vp, vp]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_rht_quantize.argtypes = [vp, i32, i64, i64, i64, u32, i32, u64, vp, vp, vp, vp, vp]
    L.nvfp4_rht_quantize.restype = i32
    L.nvfp4_quantize_row_rht.argtypes = [vp, i32, i64, i64, i64, i32, u64, vp, vp, vp, vp, u32, i32,
                                         u64, vp, vp, vp, vp, vp]
    L.nvfp4_quantize_row_rht.restype = i32
    L.mxfp4_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, u64, vp, vp, vp]
    L.mxfp4_quantize.restype = i32
    L.mxfp4_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i64, f32, vp, i64, vp]
    L.mxfp4_gemm.restype = i32
    L.nvfp4_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, i64, f32, vp, i64, vp]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_gemm_noalloc.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, i64, f32, vp]
    L.nvfp4_gemm_noalloc.restype = i32
    L.nvfp4_gemm_bf16.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, i64, f32, vp, i64,
                                  vp]
    L.nvfp4_gemm_bf16.restype = i32
    L.nvfp4_dequantize.argtypes = [vp, vp, i32, vp, i64, i64, i32, vp, i64, vp]
    L.nvfp4_dequantize.restype = i32
    L.nvfp4_gemm_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
    L.nvfp4_gemm_workspace_size.restype = i32
    L.nvfp4_set_quantize_passes.argtypes = [i32]
    L.nvfp4_set_quantize_passes.restype = i32
    L.nvfp4_set_sync_spin_limit.argtypes = [i64]
    L.nvfp4_set_sync_spin_limit.restype = i32
    L.nvfp4_single_pass_stats.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.nvfp4_single_pass_stats.restype = i32
    L.nvfp4_status_str.argtypes = [i32]
    L.nvfp4_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def _addr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def nvfp4_status_str(status: int) -> str:
    return load_library().nvfp4_status_str(status).decode()


def _check(fn: str, status: int, raise_on_error: bool) -> int:
    if status != NVFP4_OK and raise_on_error:
        raise Nvfp4Error(fn, status, nvfp4_status_str(status))
    return status


def nvfp4_quantize(x, dt, rows, cols, ld_x, layout, rnd, seed, codes, scales, codes_t,
                   scales_t, tensor_scale, amax, stream=None, raise_on_error=True) -> int:
    st = load_library().nvfp4_quantize(
        _addr(x), dt, rows, cols, ld_x, layout, rnd, seed & (2 ** 64 - 1), _addr(codes),
        _addr(scales), _addr(codes_t), _addr(scales_t), _addr(tensor_scale), _addr(amax),
        _stream(stream))
    return _check("nvfp4_quantize", st, raise_on_error)


def nvfp4_rht_quantize(x, dt, tokens, cols, ld_x, sign_mask, rnd, seed, codes, scales,
                       tensor_scale, amax, stream=None, raise_on_error=True) -> int:
    st = load_library().nvfp4_rht_quantize(
        _addr(x), dt, tokens, cols, ld_x, sign_mask & 0xFFFFFFFF, rnd, seed & (2 ** 64 - 1),
        _addr(codes), _addr(scales), _addr(tensor_scale), _addr(amax), _stream(stream))
    return _check("nvfp4_rht_quantize", st, raise_on_error)


def nvfp4_quantize_row_rht(x, dt, tokens, cols, ld_x, row_rnd, row_seed, row_codes, row_scales,
                           row_tensor_scale, row_amax, sign_mask, rht_rnd, rht_seed, rht_codes,
                           rht_scales, rht_tensor_scale, rht_amax, stream=None,
                           raise_on_error=True) -> int:
    st = load_library().nvfp4_quantize_row_rht(
        _addr(x), dt, tokens, cols, ld_x, row_rnd, row_seed & (2 ** 64 - 1), _addr(row_codes),
        _addr(row_scales), _addr(row_tensor_scale), _addr(row_amax), sign_mask & 0xFFFFFFFF,
        rht_rnd, rht_seed & (2 ** 64 - 1), _addr(rht_codes), _addr(rht_scales),
        _addr(rht_tensor_scale), _addr(rht_amax), _stream(stream))
    return _check("nvfp4_quantize_row_rht", st, raise_on_error)


def nvfp4_gemm(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_scale_rowdiv,
               b_tensor_scale, c, ldc, beta, workspace=None, workspace_bytes=None, stream=None,
               raise_on_error=True) -> int:
    """`workspace_bytes=None` takes the size of a torch-tensor workspace (0 for
    a raw address or None)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = load_library().nvfp4_gemm(
        M, N, K, _addr(a_codes), _addr(a_scales), _addr(a_tensor_scale), _addr(b_codes),
        _addr(b_scales), b_scale_rowdiv, _addr(b_tensor_scale), _addr(c), ldc, float(beta),
        _addr(workspace), int(workspace_bytes), _stream(stream))
    return _check("nvfp4_gemm", st, raise_on_error)


def nvfp4_gemm_noalloc(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes, b_scales,
                       b_scale_rowdiv, b_tensor_scale, c, ldc, beta, stream=None,
                       raise_on_error=True) -> int:
    """nvfp4_gemm with the split workspace in the library's static scratch."""
    st = load_library().nvfp4_gemm_noalloc(
        M, N, K, _addr(a_codes), _addr(a_scales), _addr(a_tensor_scale), _addr(b_codes),
        _addr(b_scales), b_scale_rowdiv, _addr(b_tensor_scale), _addr(c), ldc, float(beta),
        _stream(stream))
    return _check("nvfp4_gemm_noalloc", st, raise_on_error)


def nvfp4_gemm_bf16(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_scale_rowdiv,
                    b_tensor_scale, c, ldc, beta, workspace=None, workspace_bytes=None, stream=None,
                    raise_on_error=True) -> int:
    """nvfp4_gemm with c holding BF16 (a torch.bfloat16 tensor or its address)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = load_library().nvfp4_gemm_bf16(
        M, N, K, _addr(a_codes), _addr(a_scales), _addr(a_tensor_scale), _addr(b_codes),
        _addr(b_scales), b_scale_rowdiv, _addr(b_tensor_scale), _addr(c), ldc, float(beta),
        _addr(workspace), int(workspace_bytes), _stream(stream))
    return _check("nvfp4_gemm_bf16", st, raise_on_error)


def nvfp4_dequantize(codes, scales, scale_rowdiv, tensor_scale, rows, cols, out_dt, out, ld_out,
                     stream=None, raise_on_error=True) -> int:
    st = load_library().nvfp4_dequantize(_addr(codes), _addr(scales), scale_rowdiv,
                                         _addr(tensor_scale), rows, cols, out_dt, _addr(out),
                                         ld_out, _stream(stream))
    return _check("nvfp4_dequantize", st, raise_on_error)


def nvfp4_gemm_workspace_size(M, N, K) -> int:
    """Workspace bytes nvfp4_gemm uses for this shape on the current device."""
    out = ctypes.c_int64(0)
    _check("nvfp4_gemm_workspace_size",
           load_library().nvfp4_gemm_workspace_size(M, N, K, ctypes.byref(out)), True)
    return out.value


def mxfp4_quantize(x, dt, rows, cols, ld_x, layout, rnd, seed, codes, scales, stream=None,
                   raise_on_error=True) -> int:
    st = load_library().mxfp4_quantize(_addr(x), dt, rows, cols, ld_x, layout, rnd,
                                       seed & (2 ** 64 - 1), _addr(codes), _addr(scales),
                                       _stream(stream))
    return _check("mxfp4_quantize", st, raise_on_error)


def mxfp4_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales, c, ldc, beta, workspace=None,
               workspace_bytes=None, stream=None, raise_on_error=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = load_library().mxfp4_gemm(M, N, K, _addr(a_codes), _addr(a_scales), _addr(b_codes),
                                   _addr(b_scales), _addr(c), ldc, float(beta), _addr(workspace),
                                   int(workspace_bytes), _stream(stream))
    return _check("mxfp4_gemm", st, raise_on_error)


def nvfp4_set_quantize_passes(passes: int) -> int:
    """0: single pass where it applies (default); 2: always two passes."""
    return _check("nvfp4_set_quantize_passes", load_library().nvfp4_set_quantize_passes(passes), True)


def nvfp4_set_sync_spin_limit(polls: int) -> int:
    """Polls before a single-pass workgroup gives up waiting (tests force it)."""
    return _check("nvfp4_set_sync_spin_limit", load_library().nvfp4_set_sync_spin_limit(polls), True)


def nvfp4_single_pass_stats() -> tuple[int, int]:
    """(single-pass launches, workgroups that gave up) on the current device."""
    n, g = ctypes.c_int64(0), ctypes.c_int64(0)
    _check("nvfp4_single_pass_stats",
           load_library().nvfp4_single_pass_stats(ctypes.byref(n), ctypes.byref(g)), True)
    return n.value, g.value
