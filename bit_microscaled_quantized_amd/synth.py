"""Seeded synthetic inputs shaped like a 12B-class model's linear layers.

This module holds no NVFP4 arithmetic: it only draws seeded random tensors
(numpy PCG64 streams) and rounds FP32 draws to bf16 bit patterns.  Both the
HIP path and the CPU oracle receive the same bytes from here.

The pages report no kernel workload; the shapes follow the hidden size 5120 and
FFN size 20480 of a 12B-class layer at 8192 tokens per GPU.  Distributions:
N(0,1) with 0.1% outliers of 100*N(0,1) (activations), Student-t nu=3
(heavy-tailed Wgrad inputs), N(0, 0.02^2) weights, N(0, 1e-3^2) gradients, and
log-normal magnitudes exp(2z) with random signs (stress case).
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

_ROWS_PER_CHUNK = 1024  # fixed, so chunked draws do not depend on the thread count


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _by_rows(n_rows: int, fn) -> None:
    """fn(r0, r1) over row chunks of _ROWS_PER_CHUNK, on a thread pool (numpy
    releases the GIL inside its array loops)."""
    chunks = [(r, min(r + _ROWS_PER_CHUNK, n_rows)) for r in range(0, n_rows, _ROWS_PER_CHUNK)]
    if len(chunks) <= 1:
        for c in chunks:
            fn(*c)
        return
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda c: fn(*c), chunks))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    flat_in = x.reshape(x.shape[0], -1) if x.ndim > 1 else x.reshape(1, -1)
    flat_out = out.reshape(flat_in.shape)

    def conv(r0, r1):
        b = flat_in[r0:r1].view(np.uint32)
        lsb = (b >> np.uint32(16)) & np.uint32(1)
        flat_out[r0:r1] = ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    _by_rows(flat_in.shape[0], conv)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_with_outliers(seed: int, shape, frac: float = 1e-3, mag: float = 100.0) -> np.ndarray:
    """N(0,1) with round(frac*numel) distinct entries replaced by mag*N(0,1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    n = x.size
    k = int(round(frac * n))
    idx = rng.choice(n, size=k, replace=False)
    x.reshape(-1)[idx] = np.float32(mag) * rng.standard_normal(k, dtype=np.float32)
    return x


def token_outliers(seed: int, shape, frac: float = 1.0 / 64, mag: float = 32.0) -> np.ndarray:
    """N(0,1) rows (tokens) with round(frac*rows) distinct rows scaled by mag:
    outliers concentrated in a few tokens across every feature."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    k = int(round(frac * shape[0]))
    rows = rng.choice(shape[0], size=k, replace=False)
    x[rows] *= np.float32(mag)
    return x


def student_t(seed: int, shape, nu: float = 3.0) -> np.ndarray:
    return np.random.default_rng(seed).standard_t(nu, size=shape).astype(np.float32)


def lognormal_signed(seed: int, shape, sigma: float = 2.0) -> np.ndarray:
    """|v| = exp(sigma*z), z ~ N(0,1), with an independent random sign.  Drawn
    in chunks of 1024 rows, chunk k from the k-th child of SeedSequence(seed),
    on a thread pool (the values do not depend on the thread count)."""
    rows = shape[0]
    out = np.empty(shape, np.float32)
    kids = np.random.SeedSequence(seed).spawn(-(-rows // _ROWS_PER_CHUNK))

    def fill(r0, r1):
        rng = np.random.default_rng(kids[r0 // _ROWS_PER_CHUNK])
        sub = (r1 - r0,) + tuple(shape[1:])
        z = rng.standard_normal(sub, dtype=np.float32)
        neg = rng.integers(0, 2, size=sub, dtype=np.int8).astype(bool)
        v = np.exp(np.float32(sigma) * z)
        np.negative(v, out=v, where=neg)
        out[r0:r1] = v
    _by_rows(rows, fill)
    return out


def sign_mask16(seed: int) -> int:
    """16 random bits: bit j set means the RHT negates input j of each group."""
    return int(np.random.default_rng(seed).integers(0, 1 << 16))


def small_ints(seed: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


# --------------------------------------------------------------------------
# Workload recipes.  Each returns FP32 draws; callers convert to bf16 bits
# where the workload is bf16.
# --------------------------------------------------------------------------
HIDDEN, FFN, TOKENS = 5120, 20480, 8192

WORKLOADS = {
    "tiny_linear_256": "X, W fp32 256x256 N(0,1); X row-1D RNE, W 2D RNE; Y = X W^T",
    "quantize_sweep": "bf16 8192x5120 and 8192x20480 N(0,1) + 0.1% 100x outliers; row-1D RNE and SR",
    "wgrad_rht_5120": "dY, X bf16 8192x5120 Student-t(3); RHT column-1D (dY SR, X RNE); dW = dY^T X",
    "ffn_up_fwd_bwd": "X 8192x5120 N(0,1), W 20480x5120 N(0,0.02^2), dY 8192x20480 N(0,1e-3^2); "
                      "Fprop, Dgrad, Wgrad with RHT+SR",
    "ffn_down_stress": "X_in 32768x20480, W 5120x20480, dY 32768x5120 log-normal exp(2z) signed; "
                       "4 chunks of 8192 tokens, Wgrad accumulated",
}


def tiny_linear(seed_x: int = 1, seed_w: int = 2, n: int = 256):
    return normal(seed_x, (n, n)), normal(seed_w, (n, n))


def quantize_sweep(which: int = 0):
    if which == 0:
        return normal_with_outliers(3, (TOKENS, HIDDEN))
    return normal_with_outliers(4, (TOKENS, FFN))


def wgrad_rht(tokens: int = TOKENS, cols: int = HIDDEN):
    return dict(dy=student_t(5, (tokens, cols)), x=student_t(6, (tokens, cols)),
                sign_mask=sign_mask16(7), sr_seed=8)


def ffn_up(tokens: int = TOKENS, hidden: int = HIDDEN, ffn: int = FFN):
    return dict(x=normal(9, (tokens, hidden)), w=normal(10, (ffn, hidden), 0.02),
                dy=normal(11, (tokens, ffn), 1e-3), sign_mask=sign_mask16(12),
                sr_seed_row=13, sr_seed_col=14)


def ffn_down(tokens: int = 4 * TOKENS, hidden: int = HIDDEN, ffn: int = FFN):
    return dict(x_in=lognormal_signed(15, (tokens, ffn)), w=lognormal_signed(16, (hidden, ffn)),
                dy=lognormal_signed(17, (tokens, hidden)), sign_mask=sign_mask16(18),
                sr_seed_base=19)
