"""NVFP4 CPU oracle (ctypes shim over nvfp4_oracle.c) -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP product library neither links nor calls it; the two
share no code.  What each function computes, and which passage of the pages
(or which public format specification) it follows, is documented beside its C
definition in nvfp4_oracle.c.

Large contractions use numpy's float64 matmul (a BLAS dgemm) on the oracle's
own exactly dequantized operands; tiny ones can use the C triple loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ROW_1D, COL_1D, TILE_2D = 0, 1, 2
RNE, SR = 0, 1
BF16, F32 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile nvfp4_oracle.c into liboracle.so with plain IEEE FP32 rules."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, u64, u32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        vp, f32, f64 = ctypes.c_void_p, ctypes.c_float, ctypes.c_double
        L.ora_e2m1_value.argtypes, L.ora_e2m1_value.restype = [i32], f64
        L.ora_e4m3_value.argtypes, L.ora_e4m3_value.restype = [i32], f64
        L.ora_e4m3_rne_satfinite.argtypes, L.ora_e4m3_rne_satfinite.restype = [f32], i32
        L.ora_e2m1_rne.argtypes, L.ora_e2m1_rne.restype = [f32], i32
        L.ora_e2m1_sr.argtypes, L.ora_e2m1_sr.restype = [f32, u32], i32
        L.ora_pcg.argtypes, L.ora_pcg.restype = [u32], u32
        L.ora_sr_bits.argtypes, L.ora_sr_bits.restype = [u64, u64], u32
        L.ora_rht16.argtypes, L.ora_rht16.restype = [vp, u32, vp], None
        L.ora_encode_scale.argtypes, L.ora_encode_scale.restype = [f32], f32
        L.ora_block_scale.argtypes, L.ora_block_scale.restype = [f32, f32], i32
        L.ora_element_scale.argtypes, L.ora_element_scale.restype = [i32, f32], f32
        L.ora_block_scale_array.argtypes, L.ora_block_scale_array.restype = [vp, i64, f32, vp], None
        L.ora_quantize_range.argtypes = [vp, i32, i64, i64, i64, i32, i32, u64, vp, vp, vp, vp,
                                         vp, vp, i64, i64]
        L.ora_quantize_range.restype = i32
        L.ora_rht_quantize_range.argtypes = [vp, i32, i64, i64, i64, u32, i32, u64, vp, vp, vp,
                                             vp, i64, i64]
        L.ora_rht_quantize_range.restype = i32
        L.ora_dequant.argtypes, L.ora_dequant.restype = [i64, i64, vp, vp, i32, f32, vp], None
        L.ora_dequant_f32.argtypes, L.ora_dequant_f32.restype = [i64, i64, vp, vp, i32, f32, vp], None
        L.ora_dequant_bf16.argtypes, L.ora_dequant_bf16.restype = [i64, i64, vp, vp, i32, f32, vp], None
        L.ora_bf16_rne.argtypes, L.ora_bf16_rne.restype = [f32], ctypes.c_uint16
        L.ora_bf16_rne_array.argtypes, L.ora_bf16_rne_array.restype = [i64, vp, vp], None
        L.ora_gemm_f64.argtypes, L.ora_gemm_f64.restype = [i64, i64, i64, vp, vp, f64, vp], None
        L.ora_num_threads.argtypes, L.ora_num_threads.restype = [], i32
        L.ora_set_num_threads.argtypes, L.ora_set_num_threads.restype = [i32], None
        L.ora_mx_scale_exp.argtypes, L.ora_mx_scale_exp.restype = [f32], i32
        L.ora_mx_quantize_range.argtypes = [vp, i32, i64, i64, i64, i32, i32, u64, vp, vp, i64, i64]
        L.ora_mx_quantize_range.restype = i32
        L.ora_mx_dequant.argtypes, L.ora_mx_dequant.restype = [i64, i64, vp, vp, vp], None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ----------------------------------------------------------------- scalars
def e2m1_value(code: int) -> float:
    return lib().ora_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().ora_e4m3_value(code)


def e4m3_rne_satfinite(x: float) -> int:
    return lib().ora_e4m3_rne_satfinite(x)


def e2m1_rne(v: float) -> int:
    return lib().ora_e2m1_rne(v)


def e2m1_sr(v: float, r16: int) -> int:
    return lib().ora_e2m1_sr(v, r16)


def pcg(v: int) -> int:
    return lib().ora_pcg(v & 0xFFFFFFFF)


def sr_bits(seed: int, i: int) -> int:
    return lib().ora_sr_bits(seed, i)


def encode_scale(amax_t: float) -> float:
    return lib().ora_encode_scale(amax_t)


def block_scale(amax_b: float, s_enc: float) -> int:
    return lib().ora_block_scale(amax_b, s_enc)


def block_scale_array(amax_b: np.ndarray, s_enc: float) -> np.ndarray:
    """block_scale of every entry of an FP32 array of block maxima."""
    a = np.ascontiguousarray(amax_b, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().ora_block_scale_array(_ptr(a), a.size, s_enc, _ptr(out))
    return out


def element_scale(e_b: int, s_enc: float) -> float:
    return lib().ora_element_scale(e_b, s_enc)


def rht16(x, sign_mask: int) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(16))
    y = np.empty(16, dtype=np.float32)
    lib().ora_rht16(_ptr(x), sign_mask & 0xFFFF, _ptr(y))
    return y


def num_threads() -> int:
    return lib().ora_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the C oracle's OpenMP loops (results do not depend on it)."""
    lib().ora_set_num_threads(int(n))


# ----------------------------------------------------------------- tensors
def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16  # bf16 bit patterns
    if x.dtype == np.float32:
        return F32
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32")


def quantize(x: np.ndarray, layout: int, rnd: int = RNE, seed: int = 0,
             lines: tuple[int, int] | None = None, want_transpose: bool = True) -> dict:
    """NVFP4-quantize a 2D array (bf16 as uint16 bit patterns, or float32).

    lines = (begin, end) restricts which block lines are encoded (rows for
    ROW_1D, columns for COL_1D, 16-row tile rows for TILE_2D); the tensor amax
    is still taken over the whole tensor."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if layout == COL_1D:
        codes = np.zeros((cols, rows // 2), np.uint8)
        scales = np.zeros((cols, rows // 16), np.uint8)
    elif layout == ROW_1D:
        codes = np.zeros((rows, cols // 2), np.uint8)
        scales = np.zeros((rows, cols // 16), np.uint8)
    else:
        codes = np.zeros((rows, cols // 2), np.uint8)
        scales = np.zeros((rows // 16, cols // 16), np.uint8)
    codes_t = scales_t = None
    if layout == TILE_2D and want_transpose:
        codes_t = np.zeros((cols, rows // 2), np.uint8)
        scales_t = np.zeros((cols // 16, rows // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    am = np.zeros(1, np.float32)
    b, e = lines if lines is not None else (0, 1 << 62)
    rc = lib().ora_quantize_range(_ptr(x), _dtype_code(x), rows, cols, cols, layout, rnd,
                                  seed & ((1 << 64) - 1), _ptr(codes), _ptr(scales),
                                  _ptr(codes_t), _ptr(scales_t), _ptr(ts), _ptr(am), b, e)
    if rc != 0:
        raise ValueError(f"oracle quantize rejected shape {x.shape} layout {layout}")
    out = dict(codes=codes, scales=scales, tensor_scale=float(ts[0]), amax=float(am[0]))
    if codes_t is not None:
        out.update(codes_t=codes_t, scales_t=scales_t)
    return out


def rht_quantize(x: np.ndarray, sign_mask: int, rnd: int = RNE, seed: int = 0,
                 lines: tuple[int, int] | None = None) -> dict:
    """Random-Hadamard + column-1D NVFP4 quantization of a tokens x cols array."""
    x = np.ascontiguousarray(x)
    tokens, cols = x.shape
    codes = np.zeros((cols, tokens // 2), np.uint8)
    scales = np.zeros((cols, tokens // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    am = np.zeros(1, np.float32)
    b, e = lines if lines is not None else (0, 1 << 62)
    rc = lib().ora_rht_quantize_range(_ptr(x), _dtype_code(x), tokens, cols, cols,
                                      sign_mask & 0xFFFF, rnd, seed & ((1 << 64) - 1),
                                      _ptr(codes), _ptr(scales), _ptr(ts), _ptr(am), b, e)
    if rc != 0:
        raise ValueError(f"oracle rht_quantize rejected shape {x.shape}")
    return dict(codes=codes, scales=scales, tensor_scale=float(ts[0]), amax=float(am[0]))


def dequant(codes: np.ndarray, scales: np.ndarray, tensor_scale: float,
            scale_rowdiv: int = 1) -> np.ndarray:
    """Exact FP64 values of n x k NVFP4 codes (k contiguous)."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    n, k = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, k), np.float64)
    lib().ora_dequant(n, k, _ptr(codes), _ptr(scales), scale_rowdiv, tensor_scale, _ptr(out))
    return out


def dequant_f32(codes: np.ndarray, scales: np.ndarray, tensor_scale: float,
                scale_rowdiv: int = 1) -> np.ndarray:
    """FP32 values of n x k NVFP4 codes: the exact value rounded once."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    n, k = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, k), np.float32)
    lib().ora_dequant_f32(n, k, _ptr(codes), _ptr(scales), scale_rowdiv, tensor_scale, _ptr(out))
    return out


def dequant_bf16(codes: np.ndarray, scales: np.ndarray, tensor_scale: float,
                 scale_rowdiv: int = 1) -> np.ndarray:
    """BF16 bit patterns (uint16) of n x k NVFP4 codes: the FP32 value of
    dequant_f32 rounded to BF16, nearest even."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    n, k = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, k), np.uint16)
    lib().ora_dequant_bf16(n, k, _ptr(codes), _ptr(scales), scale_rowdiv, tensor_scale, _ptr(out))
    return out


def bf16_rne(x) -> np.ndarray:
    """BF16 bit patterns of FP32 values, nearest even (elementwise)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().ora_bf16_rne_array(x.size, _ptr(x), _ptr(out))
    return out


def mx_scale_exp(amax_b: float) -> int:
    """Shared exponent of an MXFP4 block (E8M0 code = e + 127)."""
    return lib().ora_mx_scale_exp(amax_b)


def mx_quantize(x: np.ndarray, layout: int, rnd: int = RNE, seed: int = 0,
                lines: tuple[int, int] | None = None) -> dict:
    """MXFP4-quantize a 2D array (bf16 bit patterns or float32): blocks of 32
    along rows (ROW_1D, codes [rows][cols/2], scales [rows][cols/32]) or along
    columns, written transposed (COL_1D, codes [cols][rows/2], scales
    [cols][rows/32]).  Scales are E8M0 codes; there is no tensor scale."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if layout == COL_1D:
        codes = np.zeros((cols, rows // 2), np.uint8)
        scales = np.zeros((cols, rows // 32), np.uint8)
    elif layout == ROW_1D:
        codes = np.zeros((rows, cols // 2), np.uint8)
        scales = np.zeros((rows, cols // 32), np.uint8)
    else:
        raise ValueError("MXFP4 layouts are ROW_1D and COL_1D")
    b, e = lines if lines is not None else (0, 1 << 62)
    rc = lib().ora_mx_quantize_range(_ptr(x), _dtype_code(x), rows, cols, cols, layout, rnd,
                                     seed & ((1 << 64) - 1), _ptr(codes), _ptr(scales), b, e)
    if rc != 0:
        raise ValueError(f"oracle mx_quantize rejected shape {x.shape} layout {layout}")
    return dict(codes=codes, scales=scales)


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact FP64 values of n x k MXFP4 codes (k contiguous), scales [n][k/32]."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    n, k = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, k), np.float64)
    lib().ora_mx_dequant(n, k, _ptr(codes), _ptr(scales), _ptr(out))
    return out


def gemm_f64_loop(A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None,
                  beta: float = 0.0) -> np.ndarray:
    """C = beta*C + A @ B.T by the C triple loop (tiny shapes only)."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    M, K = A.shape
    N = B.shape[0]
    out = np.zeros((M, N), np.float64) if C is None else np.array(C, np.float64, copy=True)
    lib().ora_gemm_f64(M, N, K, _ptr(A), _ptr(B), beta, _ptr(out))
    return out


def gemm_f64(A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None,
             beta: float = 0.0) -> np.ndarray:
    """C = beta*C + A @ B.T in FP64 through numpy's BLAS dgemm."""
    out = np.asarray(A, np.float64) @ np.asarray(B, np.float64).T
    if C is not None and beta != 0.0:
        out = out + beta * np.asarray(C, np.float64)
    return out
