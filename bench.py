#!/usr/bin/env python3
"""Benchmark of the NVFP4 quantize-and-contract step on one MI355X.

Headline workload: the FFN down-projection stress layer of a 12B-class model,
X_in bf16 32768x20480, W bf16 5120x20480 ([out x in]), dY bf16 32768x5120, all
with log-normal magnitudes exp(2z) and random signs.  A step quantizes W once
(16x16 2D, RNE, with its transposed copy) and then streams four chunks of 8192
tokens on one HIP stream; per chunk: X row-1D RNE together with its random
Hadamard + column-1D RNE quantization (one call), Fprop GEMM, dY row-1D SR
together with its random Hadamard + column-1D SR quantization (one call),
Dgrad GEMM with the same quantized W, Wgrad GEMM accumulated into one dW
(beta = 1 after the first chunk).  Inputs are resident in HBM before the
timed region.

Output: one JSON line.  `value` is the step's GEMM work (12 x 2MNK flops)
divided by the whole step's wall time, so quantization time counts against
it.  `roofline` describes the dominant kernel (the NVFP4 GEMM) from HIP events
around every GEMM call of the timed steps; its peak is the dense FP16 MFMA
rate, the matrix-core class the exact NVFP4 GEMM issues (the FP4 fraction is
in `components`).  `components` holds the quantize rates (HBM GB/s of the
calls' algorithmic bytes), the GEMM rates against the FP16 and FP4 peaks, the
FFN up-projection step, the quantize-only sweep timed cold (Infinity Cache
flushed by a 1 GiB read before each call), the live HBM copy rate, the MXFP4
comparison step and the autograd layer.  `cpu_baseline` times the CPU oracle
on the first chunk of the headline step, plus its quantizer single-threaded
and on all cores and its FP64 contraction.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --summarize-trace <rocprofv3 kernel_trace.csv> [--steps K --warmup W]
    python bench.py --summarize-pmc <rocprofv3 counter_collection.csv> ...
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s (% HBM peak) + NVFP4 GEMM TFLOPS (% MFMA peak), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK = 2500.0         # dense FP16 MFMA, TFLOP/s (the class the exact GEMM issues)
MFMA_FP4_PEAK = 10100.0        # dense FP4 MFMA, TFLOP/s

# headline: FFN down-projection stress layer, four chunks of 8192 tokens
S_TOKENS, S_CHUNK, S_IN, S_OUT = 32768, 8192, 20480, 5120
S_CHUNKS = S_TOKENS // S_CHUNK
# FFN up-projection layer (one 8192-token batch)
U_TOKENS, U_IN, U_OUT = 8192, 5120, 20480

# HBM bytes per k_gemm_nvfp4 launch of the headline step (mean over its
# Fprop, Dgrad and Wgrad launches), from two rocprofv3 --pmc runs (FETCH_SIZE,
# then WRITE_SIZE) of `bench.py --headline-only --copy-probe-mib 1024`, each
# scaled by what the same counter reads for the 1 GiB read + 1 GiB write
# elementwise probe.  Valid only for the kernel sources with this hash; any
# other source reports null.
GEMM_TRAFFIC = {"src_sha256": "c107f307063b53ad995bae3696362a61740c07f59d76d7b64952dd27c67b6ace",
                "bytes_per_launch": 1.2631e9}
GEMM_SOURCES = ("gemm.hip", "gemm_tiling.hpp")

GEMM_KERNEL = "k_gemm_nvfp4<float>"
REDUCE_KERNEL = "k_gemm_split_reduce<float>"


def gemm_src_sha() -> str:
    """SHA-256 over the NVFP4 GEMM kernel's sources, in GEMM_SOURCES order."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "bit_microscaled_quantized_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-sample-tokens", type=int, default=S_CHUNK)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="run only the headline step (for profiler runs)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (calibrates "
                        "the FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    p.add_argument("--summarize-pmc", nargs="+", default=None,
                   help="summarize rocprofv3 --pmc counter_collection CSVs of a "
                        "--headline-only --copy-probe-mib 1024 run and exit")
    p.add_argument("--summarize-trace", default=None,
                   help="summarize a rocprofv3 kernel-trace CSV of a bench run instead of running")
    return p.parse_args()


# ----------------------------------------------------------------- inputs
def stress_inputs():
    from bit_microscaled_quantized_amd import synth
    d = synth.ffn_down(S_TOKENS, S_OUT, S_IN)
    return dict(x=synth.f32_to_bf16_bits(d["x_in"]), w=synth.f32_to_bf16_bits(d["w"]),
                dy=synth.f32_to_bf16_bits(d["dy"]), sign_mask=d["sign_mask"],
                seed_base=d["sr_seed_base"])


def up_inputs():
    from bit_microscaled_quantized_amd import synth
    d = synth.ffn_up(U_TOKENS, U_IN, U_OUT)
    return dict(x=synth.f32_to_bf16_bits(d["x"]), w=synth.f32_to_bf16_bits(d["w"]),
                dy=synth.f32_to_bf16_bits(d["dy"]), sign_mask=d["sign_mask"],
                seed_row=d["sr_seed_row"], seed_col=d["sr_seed_col"])


def q2d_bytes(rows, cols):
    """2D quantize: input read once (bf16), codes + tile scales in both orientations."""
    n = rows * cols
    return 2 * n + 2 * (n // 2 + n // 256)


def q_row_rht_bytes(tokens, cols):
    """Fused row + RHT column quantize: input once, two sets of codes + block scales."""
    n = tokens * cols
    return 2 * n + 2 * (n // 2 + n // 16)


def q_row_bytes(rows, cols):
    n = rows * cols
    return 2 * n + n // 2 + n // 16


# ----------------------------------------------------------------- helpers
def _events_ms(torch, fn, steps, warmup):
    """Mean HIP-event time of fn() on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


class Timer:
    """Collects (name, start, end) HIP events around calls on the current stream."""

    def __init__(self, torch, on: bool):
        self.torch, self.on, self.rec = torch, on, []

    def __call__(self, name, fn):
        if not self.on:
            fn()
            return
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.rec.append((name, a, b))

    def means(self):
        per = {}
        for name, a, b in self.rec:
            per.setdefault(name, []).append(a.elapsed_time(b))
        return {k: float(np.mean(v)) for k, v in per.items()}, per


def run_steps(torch, step, steps, warmup):
    """Warmup, then K steps between two synchronizations (wall time), then K
    more with HIP events around every call.  Returns (ms per step, per-call
    mean ms, per-call lists)."""
    off = Timer(torch, False)
    for _ in range(warmup):
        step(off)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(off)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    tm = Timer(torch, True)
    for _ in range(steps):
        step(tm)
    torch.cuda.synchronize()
    per, lists = tm.means()
    return wall * 1e3, per, lists


# ----------------------------------------------------------------- headline
def stress_bench(torch, nv, inp, steps, warmup):
    """The headline step; returns its figures and the device tensors."""
    from bit_microscaled_quantized_amd.linear import LinearStep
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev)

    x, w, dy = up(inp["x"]), up(inp["w"]), up(inp["dy"])
    T, I, O = S_CHUNK, S_IN, S_OUT
    st = LinearStep(T, I, O, device=dev)
    bf, RNE, SR = nv.NVFP4_BF16, nv.NVFP4_RNE, nv.NVFP4_SR
    mask, base = inp["sign_mask"], inp["seed_base"]
    qw, qx, qxt, qd, qdt = st.qw, st.qx, st.qx_t, st.qdy, st.qdy_t
    xs = [x[c * T:(c + 1) * T] for c in range(S_CHUNKS)]
    dys = [dy[c * T:(c + 1) * T] for c in range(S_CHUNKS)]

    def step(tm):
        tm("quant_w_2d", lambda: nv.nvfp4_quantize(
            w, bf, O, I, I, nv.NVFP4_TILE_2D, RNE, 0, qw.codes, qw.scales, qw.codes_t, qw.scales_t,
            qw.ts, qw.amax))
        for c in range(S_CHUNKS):
            xc, dc = xs[c], dys[c]
            tm("quant_x_row_rht", lambda: nv.nvfp4_quantize_row_rht(
                xc, bf, T, I, I, RNE, 0, qx.codes, qx.scales, qx.ts, qx.amax, mask,
                RNE, 0, qxt.codes, qxt.scales, qxt.ts, qxt.amax))
            tm("gemm_fprop", lambda: nv.nvfp4_gemm(
                T, O, I, qx.codes, qx.scales, qx.ts, qw.codes, qw.scales, 16, qw.ts, st.y, O, 0.0,
                workspace=st.ws))
            s_row, s_col = base + 2 * c, base + 2 * c + 1
            tm("quant_dy_row_rht_sr", lambda: nv.nvfp4_quantize_row_rht(
                dc, bf, T, O, O, SR, s_row, qd.codes, qd.scales, qd.ts, qd.amax, mask,
                SR, s_col, qdt.codes, qdt.scales, qdt.ts, qdt.amax))
            tm("gemm_dgrad", lambda: nv.nvfp4_gemm(
                T, I, O, qd.codes, qd.scales, qd.ts, qw.codes_t, qw.scales_t, 16, qw.ts, st.dx, I,
                0.0, workspace=st.ws))
            beta = 1.0 if c > 0 else 0.0
            tm("gemm_wgrad", lambda: nv.nvfp4_gemm(
                O, I, T, qdt.codes, qdt.scales, qdt.ts, qxt.codes, qxt.scales, 1, qxt.ts, st.dw, I,
                beta, workspace=st.ws))

    ms_step, per, lists = run_steps(torch, step, steps, warmup)
    gemm_calls = lists["gemm_fprop"] + lists["gemm_dgrad"] + lists["gemm_wgrad"]
    flops = 2.0 * T * I * O
    q_ms = per["quant_w_2d"] + S_CHUNKS * (per["quant_x_row_rht"] + per["quant_dy_row_rht_sr"])
    q_bytes = q2d_bytes(O, I) + S_CHUNKS * (q_row_rht_bytes(T, I) + q_row_rht_bytes(T, O))
    out = dict(ms_step=ms_step, per=per, gemm_ms=float(np.mean(gemm_calls)), gemm_flops=flops,
               gemm_launches=len(gemm_calls), q_ms=q_ms, q_bytes=q_bytes,
               q_bytes_by_call={"quant_w_2d": q2d_bytes(O, I),
                                "quant_x_row_rht": q_row_rht_bytes(T, I),
                                "quant_dy_row_rht_sr": q_row_rht_bytes(T, O)})
    del x, w, dy, st, xs, dys
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------- FFN up
def up_bench(torch, nv, inp, steps, warmup):
    """The FFN up-projection layer's step (one 8192-token batch, W quantized
    every step), as in the headline but with one chunk."""
    from bit_microscaled_quantized_amd.linear import LinearStep
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev)

    x, w, dy = up(inp["x"]), up(inp["w"]), up(inp["dy"])
    T, I, O = U_TOKENS, U_IN, U_OUT
    st = LinearStep(T, I, O, device=dev)
    bf, RNE, SR = nv.NVFP4_BF16, nv.NVFP4_RNE, nv.NVFP4_SR
    mask, s_row, s_col = inp["sign_mask"], inp["seed_row"], inp["seed_col"]
    qw, qx, qxt, qd, qdt = st.qw, st.qx, st.qx_t, st.qdy, st.qdy_t

    def step(tm):
        tm("quant_x_row_rht", lambda: nv.nvfp4_quantize_row_rht(
            x, bf, T, I, I, RNE, 0, qx.codes, qx.scales, qx.ts, qx.amax, mask,
            RNE, 0, qxt.codes, qxt.scales, qxt.ts, qxt.amax))
        tm("quant_w_2d", lambda: nv.nvfp4_quantize(
            w, bf, O, I, I, nv.NVFP4_TILE_2D, RNE, 0, qw.codes, qw.scales, qw.codes_t, qw.scales_t,
            qw.ts, qw.amax))
        tm("gemm_fprop", lambda: nv.nvfp4_gemm(
            T, O, I, qx.codes, qx.scales, qx.ts, qw.codes, qw.scales, 16, qw.ts, st.y, O, 0.0,
            workspace=st.ws))
        tm("quant_dy_row_rht_sr", lambda: nv.nvfp4_quantize_row_rht(
            dy, bf, T, O, O, SR, s_row, qd.codes, qd.scales, qd.ts, qd.amax, mask,
            SR, s_col, qdt.codes, qdt.scales, qdt.ts, qdt.amax))
        tm("gemm_dgrad", lambda: nv.nvfp4_gemm(
            T, I, O, qd.codes, qd.scales, qd.ts, qw.codes_t, qw.scales_t, 16, qw.ts, st.dx, I, 0.0,
            workspace=st.ws))
        tm("gemm_wgrad", lambda: nv.nvfp4_gemm(
            O, I, T, qdt.codes, qdt.scales, qdt.ts, qxt.codes, qxt.scales, 1, qxt.ts, st.dw, I, 0.0,
            workspace=st.ws))

    ms_step, per, _ = run_steps(torch, step, steps, warmup)
    flops = 2.0 * T * I * O
    gemm_ms = float(np.mean([per["gemm_fprop"], per["gemm_dgrad"], per["gemm_wgrad"]]))
    qb = {"quant_x_row_rht": q_row_rht_bytes(T, I), "quant_w_2d": q2d_bytes(O, I),
          "quant_dy_row_rht_sr": q_row_rht_bytes(T, O)}
    q_ms = sum(per[k] for k in qb)
    q_gbs = sum(qb.values()) / (q_ms * 1e-3) / 1e9
    gt = flops / (gemm_ms * 1e-3) / 1e12
    mx = mx_bench(torch, nv, x, w, dy, s_row, s_col, steps, warmup)
    mod = module_bench(torch, nv, x, w, dy, st, steps, warmup)
    out = {
        "workload": "ffn_up_fwd_bwd: X bf16 8192x5120 N(0,1), W bf16 20480x5120 N(0,0.02^2), "
                    "dY bf16 8192x20480 N(0,1e-3^2); same calls as the headline, one chunk, "
                    "W quantized every step",
        "ms_per_step": round(ms_step, 4),
        "TFLOPs": round(3 * flops / (ms_step * 1e-3) / 1e12, 2),
        "quantize_GBps": round(q_gbs, 1),
        "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
        "gemm_TFLOPs": round(gt, 2),
        "gemm_frac_mfma_f16": round(gt / MFMA_F16_PEAK, 4),
        "per_call_ms": {k: round(v, 4) for k, v in per.items()},
        "quantize_bytes": qb,
        "mxfp4": mx,
        "linear_module": mod,
    }
    del x, w, dy, st
    torch.cuda.empty_cache()
    return out


def copy_bench(torch, mib=1024, steps=10, warmup=3):
    """Achievable HBM rate on this GPU: an elementwise kernel (torch.neg) that
    reads and writes `mib` MiB each, read + write bytes per second (GB/s)."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = _events_ms(torch, lambda: torch.neg(src, out=dst), steps, warmup)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (mib << 20) / (ms * 1e-3) / 1e9


def module_bench(torch, nv, x, w, dy, st, steps, warmup):
    """The autograd layer on the FFN up-projection tensors: NVFP4Linear forward
    + backward (quantize, Fprop, Dgrad, Wgrad, BF16 outputs) against the same
    layer kept in BF16 (torch's BF16 matmul); and NVFP4 -> BF16 dequantization
    of W."""
    from bit_microscaled_quantized_amd.module import NVFP4Linear
    T, I, O = U_TOKENS, U_IN, U_OUT
    xb = x.view(torch.bfloat16)
    dyb = dy.view(torch.bfloat16)
    out = {}
    for name, bypass in (("nvfp4", False), ("bf16", True)):
        layer = NVFP4Linear(I, O, bf16=bypass, seed=1, device=x.device)
        with torch.no_grad():
            layer.weight.copy_(w.view(torch.bfloat16))
        xi = xb.detach().clone().requires_grad_(True)

        def fwd_bwd():
            layer.weight.grad = None
            xi.grad = None
            layer(xi).backward(dyb)
        ms = _events_ms(torch, fwd_bwd, steps, warmup)
        out[f"{name}_fwd_bwd_ms"] = round(ms, 4)
        out[f"{name}_TFLOPs"] = round(3 * 2.0 * T * I * O / (ms * 1e-3) / 1e12, 2)
    q = st.qw  # W quantized by the step above
    wd = torch.empty((O, I), dtype=torch.bfloat16, device=x.device)
    ms = _events_ms(torch, lambda: nv.nvfp4_dequantize(q.codes, q.scales, 16, q.ts, O, I, nv.NVFP4_BF16,
                                                       wd, I), steps, warmup)
    nbytes = O * I // 2 + O * I // 256 + O * I * 2
    out["dequant_w_bf16_ms"] = round(ms, 4)
    out["dequant_w_bf16_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["dequant_frac_hbm"] = round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    return out


def mx_bench(torch, nv, x, w, dy, s_row, s_col, steps, warmup):
    """The MXFP4 comparison step on the FFN up-projection tensors: each of the
    six quantize calls (bf16 in, codes + E8M0 scales out) and three GEMMs timed
    with HIP events on the current stream."""
    dev = x.device
    T, I, O = U_TOKENS, U_IN, U_OUT
    bf = nv.NVFP4_BF16
    u8 = dict(dtype=torch.uint8, device=dev)

    def buf(rows, cols):  # codes and scales of `rows` lines of `cols` elements
        return torch.empty((rows, cols // 2), **u8), torch.empty((rows, cols // 32), **u8)
    w_r, w_c = buf(O, I), buf(I, O)
    x_r, x_c = buf(T, I), buf(I, T)
    d_r, d_c = buf(T, O), buf(O, T)
    y = torch.empty((T, O), dtype=torch.float32, device=dev)
    dx = torch.empty((T, I), dtype=torch.float32, device=dev)
    dw = torch.empty((O, I), dtype=torch.float32, device=dev)
    ws = torch.empty((max(nv.nvfp4_gemm_workspace_size(T, O, I), nv.nvfp4_gemm_workspace_size(T, I, O),
                          nv.nvfp4_gemm_workspace_size(O, I, T), 4) // 4,), dtype=torch.float32, device=dev)
    R, C, RNE, SR = nv.NVFP4_ROW_1D, nv.NVFP4_COL_1D, nv.NVFP4_RNE, nv.NVFP4_SR
    calls = [
        ("w_row", lambda: nv.mxfp4_quantize(w, bf, O, I, I, R, RNE, 0, *w_r)),
        ("w_col", lambda: nv.mxfp4_quantize(w, bf, O, I, I, C, RNE, 0, *w_c)),
        ("x_row", lambda: nv.mxfp4_quantize(x, bf, T, I, I, R, RNE, 0, *x_r)),
        ("x_col", lambda: nv.mxfp4_quantize(x, bf, T, I, I, C, RNE, 0, *x_c)),
        ("gemm_fprop", lambda: nv.mxfp4_gemm(T, O, I, *x_r, *w_r, y, O, 0.0, workspace=ws)),
        ("dy_row_sr", lambda: nv.mxfp4_quantize(dy, bf, T, O, O, R, SR, s_row, *d_r)),
        ("dy_col_sr", lambda: nv.mxfp4_quantize(dy, bf, T, O, O, C, SR, s_col, *d_c)),
        ("gemm_dgrad", lambda: nv.mxfp4_gemm(T, I, O, *d_r, *w_c, dx, I, 0.0, workspace=ws)),
        ("gemm_wgrad", lambda: nv.mxfp4_gemm(O, I, T, *d_c, *x_c, dw, I, 0.0, workspace=ws)),
    ]

    def step(tm):
        for name, fn in calls:
            tm(name, fn)
    _, per, _ = run_steps(torch, step, steps, warmup)

    def one(n):
        return n * 2 + n // 2 + n // 32
    qb = dict(w_row=one(O * I), w_col=one(O * I), x_row=one(T * I), x_col=one(T * I),
              dy_row_sr=one(T * O), dy_col_sr=one(T * O))
    q_ms = sum(per[k] for k in qb)
    g_ms = float(np.mean([per["gemm_fprop"], per["gemm_dgrad"], per["gemm_wgrad"]]))
    g_tf = 2.0 * T * I * O / (g_ms * 1e-3) / 1e12
    q_gbs = sum(qb.values()) / (q_ms * 1e-3) / 1e9
    return {
        "quantize_GBps": round(q_gbs, 1),
        "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
        "gemm_TFLOPs": round(g_tf, 2),
        "gemm_frac_mfma_fp4": round(g_tf / MFMA_FP4_PEAK, 4),
        "step_ms": round(sum(per.values()), 4),
        "per_call_ms": {k: round(v, 4) for k, v in per.items()},
        "quantize_bytes": qb,
    }


# ----------------------------------------------------------------- quantize-only sweep
def sweep_bench(torch, nv, steps):
    """The quantize-only workload, each call timed cold: bf16 tensors 8192x5120
    and 8192x20480 (N(0,1) with 0.1% 100x outliers), row-1D, RNE and SR, one
    nvfp4_quantize call each.  Before every timed call a 1 GiB read (outside
    the events) evicts the tensor from the 256 MB Infinity Cache.  GB/s counts
    the call's algorithmic bytes: input read once (2 B/elem), codes
    (0.5 B/elem) and E4M3 scales (1/16 B/elem); the median over the calls is
    reported."""
    from bit_microscaled_quantized_amd import synth
    dev = torch.device("cuda", 0)
    u8 = dict(dtype=torch.uint8, device=dev)
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    out = {}
    for which in (0, 1):
        xb = synth.f32_to_bf16_bits(synth.quantize_sweep(which))
        R, C = xb.shape
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        codes, scales = torch.empty((R, C // 2), **u8), torch.empty((R, C // 16), **u8)
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        am = torch.empty(1, dtype=torch.float32, device=dev)
        nbytes = q_row_bytes(R, C)
        for rname, rnd, seed in (("rne", nv.NVFP4_RNE, 0), ("sr", nv.NVFP4_SR, 3)):
            def call():
                nv.nvfp4_quantize(x, nv.NVFP4_BF16, R, C, C, nv.NVFP4_ROW_1D, rnd, seed, codes,
                                  scales, None, None, ts, am)
            for _ in range(3):
                call()
            times = []
            for _ in range(max(steps, 5)):
                torch.amax(flush, dim=0, out=sink)  # a 1 GiB read evicts the Infinity Cache
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
            ms = float(np.median(times))
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[f"{R}x{C}_{rname}"] = dict(ms=round(ms, 4), GBps=round(gbs, 1),
                                          frac_hbm=round(gbs / HBM_PEAK_GBS, 4), bytes=nbytes)
        del x, codes, scales
        torch.cuda.empty_cache()
    tot_b = sum(v["bytes"] for v in out.values())
    tot_ms = sum(v["ms"] for v in out.values())
    out["all"] = dict(GBps=round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
                      frac_hbm=round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    out["timing"] = "cold: a 1 GiB read before each call, median of the calls"
    del flush
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------- CPU baseline
def cpu_baseline(inp, tokens):
    """The oracle, as it stands, on the first `tokens` tokens of the headline
    step (its first chunk) with the full weight: W 2D, X row + RHT, dY row SR +
    RHT SR quantization in C (OpenMP over blocks, all host threads) and the
    three FP64 contractions of the dequantized operands (numpy BLAS).  Also the
    oracle's row-1D quantizer alone on one thread and on all threads, and one
    FP64 contraction, each with its thread count."""
    import oracle as ora
    from threadpoolctl import threadpool_info
    x, w, dy = inp["x"][:tokens], inp["w"], inp["dy"][:tokens]
    mask, base = inp["sign_mask"], inp["seed_base"]
    threads = ora.num_threads()
    t0 = time.perf_counter()
    qw = ora.quantize(w, ora.TILE_2D, ora.RNE)
    qx = ora.quantize(x, ora.ROW_1D, ora.RNE)
    qxt = ora.rht_quantize(x, mask, ora.RNE)
    dqx = ora.dequant(qx["codes"], qx["scales"], qx["tensor_scale"])
    dqw = ora.dequant(qw["codes"], qw["scales"], qw["tensor_scale"], 16)
    tq = time.perf_counter()
    y = ora.gemm_f64(dqx, dqw)
    tg = time.perf_counter() - tq
    del dqx, dqw
    qd = ora.quantize(dy, ora.ROW_1D, ora.SR, base)
    qdt = ora.rht_quantize(dy, mask, ora.SR, base + 1)
    dx = ora.gemm_f64(ora.dequant(qd["codes"], qd["scales"], qd["tensor_scale"]),
                      ora.dequant(qw["codes_t"], qw["scales_t"], qw["tensor_scale"], 16))
    dw = ora.gemm_f64(ora.dequant(qdt["codes"], qdt["scales"], qdt["tensor_scale"]),
                      ora.dequant(qxt["codes"], qxt["scales"], qxt["tensor_scale"]))
    dt = time.perf_counter() - t0
    del y, dx, dw
    flops = 3 * 2.0 * tokens * S_IN * S_OUT
    blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])

    # the row-1D quantizer alone (RNE, bf16), all threads, then one thread on a
    # sixteenth of the rows
    xs = inp["x"][:tokens]
    nb = q_row_bytes(*xs.shape)
    t1 = time.perf_counter()
    ora.quantize(xs, ora.ROW_1D, ora.RNE)
    q_all = nb / (time.perf_counter() - t1) / 1e9
    ora.set_num_threads(1)
    xs1 = xs[: tokens // 16]
    t1 = time.perf_counter()
    ora.quantize(xs1, ora.ROW_1D, ora.RNE)
    q_one = q_row_bytes(*xs1.shape) / (time.perf_counter() - t1) / 1e9
    ora.set_num_threads(threads)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=max(threads, blas), kind="oracle",
                seconds=round(dt, 3),
                sample=f"the headline step's first chunk ({tokens} of {S_TOKENS} tokens) with the full "
                       f"{S_OUT}x{S_IN} weight: W 2D, X row + RHT, dY row SR + RHT SR quantization in "
                       f"the C oracle (OpenMP, {threads} threads) + 3 FP64 BLAS contractions "
                       f"({blas} threads); value = that chunk's 3 x 2MNK flops / its wall time",
                quantize_row_GBps_all_threads=round(q_all, 3), quantize_threads=threads,
                quantize_row_GBps_one_thread=round(q_one, 3),
                gemm_f64_GFLOPs=round(2.0 * tokens * S_IN * S_OUT / tg / 1e9, 1), gemm_threads=blas)


# ----------------------------------------------------------------- trace summary
def _kernel_short(name: str) -> str:
    s = name.replace("(anonymous namespace)::", "").split("(")[0]
    return s.replace("void ", "").replace("nvfp4::", "").strip()


def summarize_trace(path, steps, warmup):
    """Markdown summary of a rocprofv3 kernel-trace CSV of `bench.py` with the
    same --steps / --warmup: per-kernel statistics over the whole run, and the
    NVFP4 GEMM launches of the headline's timed steps (the first `warmup`
    steps' launches skipped, the next 2 x `steps` steps' taken: wall-timed
    and event-timed), each with the split-tail reduction that follows it."""
    rows, grids = [], []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                         _kernel_short(r["Kernel_Name"])))
            grids.append((int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1),
                          int(r["Grid_Size_Y"]) // max(int(r["Workgroup_Size_Y"]), 1)))
    order = sorted(range(len(rows)), key=lambda i: rows[i])
    rows = [rows[i] for i in order]
    grids = [grids[i] for i in order]
    stats = {}
    for i, ((s, e, k), g) in enumerate(zip(rows, grids)):
        nxt = f"{rows[i + 1][2]} {grids[i + 1][0]}x{grids[i + 1][1]}" if i + 1 < len(rows) else None
        stats.setdefault((_with_next(k, nxt), g), []).append((e - s) / 1e3)
    total = sum(sum(v) for v in stats.values())
    print("| kernel | grid (workgroups x by y) | calls | mean µs | median µs | total ms | % of kernel time |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for (k, g), v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        name = k if len(k) <= 90 else k[:87] + "..."
        print(f"| `{name}` | {g[0]}x{g[1]} | {len(v)} | {np.mean(v):.1f} | {np.median(v):.1f} | "
              f"{sum(v) / 1e3:.3f} | {100 * sum(v) / total:.1f} |")
    per_step = 3 * S_CHUNKS
    gem = [(i, s, e) for i, (s, e, k) in enumerate(rows) if k == GEMM_KERNEL]
    first, n = warmup * per_step, 2 * steps * per_step
    timed = gem[first:first + n]
    if len(timed) < n:
        print(f"\nonly {len(timed)} of {n} headline GEMM launches found")
        return
    dur, call = [], []
    for i, s, e in timed:
        d = (e - s) / 1e3
        extra = 0.0
        j = i + 1
        if j < len(rows) and rows[j][2] == REDUCE_KERNEL:
            extra = (rows[j][1] - rows[j][0]) / 1e3
        dur.append(d)
        call.append(d + extra)
    flops = 2.0 * S_CHUNK * S_IN * S_OUT
    km, cm = float(np.mean(dur)), float(np.mean(call))
    print(f"\nheadline timed-region `{GEMM_KERNEL}` launches: {len(dur)}")
    print(f"- kernel alone: mean {km:.1f} µs -> {flops / km / 1e6:.1f} TFLOP/s = "
          f"{flops / km / 1e6 / MFMA_F16_PEAK:.4f} of the FP16 MFMA peak")
    print(f"- kernel + its split-tail reduction (what one nvfp4_gemm call takes): mean {cm:.1f} µs "
          f"-> {flops / cm / 1e6:.1f} TFLOP/s = {flops / cm / 1e6 / MFMA_F16_PEAK:.4f}")
    for name, sl in (("Fprop", slice(0, None, 3)), ("Dgrad", slice(1, None, 3)),
                     ("Wgrad", slice(2, None, 3))):
        d = dur[sl]
        print(f"- {name}: {len(d)} launches, mean {np.mean(d):.1f} µs, median {np.median(d):.1f} µs")


def _with_next(k, nxt):
    """An amax pass is told apart by the cast that follows it, named with its
    grid (passes over tensors of different sizes can share one grid: a
    resident grid)."""
    if nxt is not None and (k.startswith("k_rht_amax") or k.startswith("k_amax")):
        return f"{k} -> {nxt}"
    return k


# ----------------------------------------------------------------- counter summary
def _headline_labels():
    """(short kernel name, workgroups) -> (label, algorithmic bytes read, written)
    for the launches of one headline step on a 256-CU device; the Wgrad
    figures average its beta = 0 launch and its three beta = 1 launches.  An
    amax pass is keyed by "<kernel> -> <the kernel after it>" and any grid
    (None)."""
    T, I, O = S_CHUNK, S_IN, S_OUT

    def q_out(rows, cols):  # codes + scales of one NVFP4 copy
        return rows * cols // 2 + rows * cols // 16

    w_in, x_in, d_in = O * I * 2, T * I * 2, T * O * 2
    wg_acc = 0.75 * O * I * 4
    return {
        (f"k_amax<unsigned short, 8> -> k_cast_tile2d<unsigned short, 0> {(O // 256) * (I // 64)}", None):
            ("W amax (5120x20480)", w_in, 0),
        ("k_cast_tile2d<unsigned short, 0>", (O // 256) * (I // 64)):
            ("W 2D cast + transposed copy", w_in, 2 * q_out(O, I) - 2 * (O * I // 16) + 2 * (O * I // 256)),
        (f"k_rht_amax<unsigned short> -> k_cast_row_rht<unsigned short, 0, 0> {(I // 128) * (T // 256)}", None):
            ("X RHT + plain amax (8192x20480)", x_in, 0),
        ("k_cast_row_rht<unsigned short, 0, 0>", (I // 128) * (T // 256)):
            ("X row + RHT column cast, RNE", x_in, 2 * q_out(T, I)),
        (f"k_rht_amax<unsigned short> -> k_cast_row_rht<unsigned short, 1, 1> {(O // 128) * (T // 256)}", None):
            ("dY RHT + plain amax (8192x5120)", d_in, 0),
        ("k_cast_row_rht<unsigned short, 1, 1>", (O // 128) * (T // 256)):
            ("dY row + RHT column cast, SR", d_in, 2 * q_out(T, O)),
        ("k_gemm_nvfp4<float>", 768): ("Fprop 8192x5120x20480", q_out(T, I) + O * I // 2 + O * I // 256,
                                       T * O * 4),
        ("k_gemm_nvfp4<float>", 2560): ("Dgrad 8192x20480x5120", q_out(T, O) + O * I // 2 + O * I // 256,
                                        T * I * 4),
        ("k_gemm_nvfp4<float>", 1792): ("Wgrad 5120x20480x8192 (3 of 4 with beta = 1)",
                                        q_out(O, T) + q_out(I, T) + wg_acc, O * I * 4),
    }


def summarize_pmc(paths):
    """Markdown summary of rocprofv3 --pmc counter_collection CSVs of
    `bench.py --headline-only --copy-probe-mib 1024`: per kernel and grid the
    mean counter values per dispatch; FETCH_SIZE / WRITE_SIZE scaled by what
    they read for the copy probe (reads and writes 1 GiB) and set against the
    launch's algorithmic bytes; VALU instructions per element for the
    quantize kernels."""
    groups = {}
    for path in paths:
        with open(path) as f:
            recs = list(csv.DictReader(f))
        names = {int(r["Dispatch_Id"]): f'{_kernel_short(r["Kernel_Name"])} '
                 f'{int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)}' for r in recs}
        for r in recs:
            wgs = int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)
            d = int(r["Dispatch_Id"])
            key = (_with_next(_kernel_short(r["Kernel_Name"]), names.get(d + 1)), wgs)
            g = groups.setdefault(key, {})
            g.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
    probe = [g for (k, _), g in groups.items() if "neg_kernel" in k]
    gib_kib = float(1 << 20)
    fetch_f = write_f = None
    if probe:
        if "FETCH_SIZE" in probe[0]:
            fetch_f = gib_kib / np.mean(list(probe[0]["FETCH_SIZE"].values()))
        if "WRITE_SIZE" in probe[0]:
            write_f = gib_kib / np.mean(list(probe[0]["WRITE_SIZE"].values()))
    print("Calibration (copy probe: 1 GiB read, 1 GiB written): "
          f"FETCH_SIZE factor {fetch_f if fetch_f is None else round(fetch_f, 3)}, "
          f"WRITE_SIZE factor {write_f if write_f is None else round(write_f, 3)}\n")
    labels = _headline_labels()
    elems = {"W": S_OUT * S_IN, "X": S_CHUNK * S_IN, "dY": S_CHUNK * S_OUT}
    print("| kernel | workgroups | launch | dispatches | FETCH KiB | WRITE KiB | HBM MB read / written "
          "| algorithmic MB read / written | HBM / algorithmic | VALU per element |")
    print("|---|---:|---|---:|---:|---:|---:|---:|---:|---:|")
    gemm_bytes, gemm_n = 0.0, 0
    for (k, wgs), g in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        if not (k.startswith("k_") or "neg_kernel" in k):
            continue
        n = max(len(v) for v in g.values())
        fk = np.mean(list(g["FETCH_SIZE"].values())) if "FETCH_SIZE" in g else None
        wk = np.mean(list(g["WRITE_SIZE"].values())) if "WRITE_SIZE" in g else None
        rd = fk * 1024 * fetch_f if fk is not None and fetch_f else None
        wr = wk * 1024 * write_f if wk is not None and write_f else None
        lab, ar, aw = labels.get((k, wgs), labels.get((k, None), ("", None, None)))
        ratio = ""
        if rd is not None and wr is not None and ar is not None:
            ratio = f"{(rd + wr) / (ar + aw):.2f}"
            if k == GEMM_KERNEL:
                gemm_bytes += (rd + wr) * n
                gemm_n += n
        valu = ""
        if "SQ_INSTS_VALU" in g and lab[:2] in ("W ", "X ", "dY"):
            e = elems[lab.split()[0]]
            valu = f"{np.mean(list(g['SQ_INSTS_VALU'].values())) * 64 / e:.1f}"
        f = lambda v, d=0: "" if v is None else f"{v:.{d}f}"
        amb = "" if ar is None else f"{ar / 1e6:.1f} / {aw / 1e6:.1f}"
        hbm = "" if rd is None or wr is None else f"{rd / 1e6:.1f} / {wr / 1e6:.1f}"
        print(f"| `{k}` | {wgs} | {lab} | {n} | {f(fk)} | {f(wk)} | {hbm} | {amb} | {ratio} | {valu} |")
    if gemm_n:
        print(f"\n`{GEMM_KERNEL}`: mean HBM bytes per launch over {gemm_n} headline launches: "
              f"{gemm_bytes / gemm_n:.4e} (sources sha256 {gemm_src_sha()})")
    sq = [(k, g) for k, g in groups.items() if k[0] == GEMM_KERNEL and "SQ_INSTS_MFMA" in g]
    for (k, wgs), g in sq:
        m = {c: np.mean(list(v.values())) for c, v in g.items()}
        line = ", ".join(f"{c} {v:.4g}" for c, v in sorted(m.items()))
        print(f"- `{k}` {wgs} workgroups ({labels.get((k, wgs), ('',))[0]}): {line}")


# ----------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps, args.warmup)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sharded path is a design, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_microscaled_quantized_amd as nv
    nv.load_library()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)

    inp = stress_inputs()
    head = stress_bench(torch, nv, inp, args.steps, args.warmup)
    comps = {}
    if not args.headline_only:
        comps["ffn_up"] = up_bench(torch, nv, up_inputs(), args.steps, args.warmup)
        comps["quantize_sweep"] = sweep_bench(torch, nv, args.steps)
        comps["hbm_copy_GBps"] = round(copy_bench(torch), 1)
    if args.copy_probe_mib:
        # an elementwise kernel (not a DMA copy, which no counter sees) that
        # reads and writes exactly n bytes
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    flops = head["gemm_flops"]
    ms_step = head["ms_step"]
    gemm_ms = head["gemm_ms"]
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    q_gbs = head["q_bytes"] / (head["q_ms"] * 1e-3) / 1e9
    value = 3 * S_CHUNKS * flops / (ms_step * 1e-3) / 1e12
    traffic = None
    if GEMM_TRAFFIC is not None and GEMM_TRAFFIC["src_sha256"] == gemm_src_sha():
        traffic = GEMM_TRAFFIC["bytes_per_launch"]
    per = head["per"]
    comps.update({
        "quantize_GBps": round(q_gbs, 1),
        "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
        "quantize_bytes_per_call": head["q_bytes_by_call"],
        "quantize_GBps_per_call": {k: round(b / (per[k] * 1e-3) / 1e9, 1)
                                   for k, b in head["q_bytes_by_call"].items()},
        "gemm_TFLOPs": round(gemm_tflops, 2),
        "gemm_frac_mfma_f16": round(gemm_tflops / MFMA_F16_PEAK, 4),
        "gemm_frac_mfma_fp4": round(gemm_tflops / MFMA_FP4_PEAK, 4),
        "per_call_ms": {k: round(v, 4) for k, v in per.items()},
    })
    if "hbm_copy_GBps" in comps:
        comps["quantize_frac_of_copy"] = round(q_gbs / comps["hbm_copy_GBps"], 4)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "ffn_down_stress: X_in bf16 32768x20480, W bf16 5120x20480 [out x in], "
                        "dY bf16 32768x5120, log-normal |v| = exp(2z) with random signs; W 2D RNE "
                        "(+transposed) once; 4 chunks of 8192 tokens on one stream, each: X row RNE "
                        "+ RHT col RNE, Fprop, dY row SR + RHT col SR, Dgrad, Wgrad (beta = 1 after "
                        "the first chunk)",
            "tokens": S_TOKENS, "chunk_tokens": S_CHUNK, "d_in": S_IN, "d_out": S_OUT,
        },
        "roofline": {
            "kernel": "k_gemm_nvfp4",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": MFMA_F16_PEAK,
            "peak_kind": "dense FP16 MFMA: the exact NVFP4 GEMM dequantizes to FP16 and issues "
                         "FP16 MFMAs; the FP4-peak fraction is components.gemm_frac_mfma_fp4",
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / MFMA_F16_PEAK, 4),
            "traffic": traffic,
            "avg_launch_ms": round(gemm_ms, 4),
            "launches": head["gemm_launches"],
            "flops_per_launch": flops,
        },
        "components": comps,
    }
    if not args.no_cpu_baseline and not args.headline_only:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
