#!/usr/bin/env python3
"""Benchmark of the NVFP4 quantize-and-contract step of one linear layer on
one MI355X.

A step is the whole hot path over one batch of the FFN up-projection layer
(X bf16 8192x5120, W bf16 20480x5120 ~N(0, 0.02^2), dY bf16 8192x20480
~N(0, 1e-3^2)): X row-1D RNE together with its random Hadamard + column-1D
quantization (RNE, the Wgrad operand) in one call; W 16x16 2D quantize (RNE,
with the transposed copy); Fprop GEMM; dY row-1D SR together with its random
Hadamard + column-1D SR quantization in one call; Dgrad GEMM with the same
quantized W; Wgrad GEMM.  Inputs are resident in HBM before the timed region.

Output: one JSON line.  `value` is the step's GEMM work (3 x 2MNK flops)
divided by the whole step's wall time, so quantization time counts against
it; the per-component figures (quantize GB/s, GEMM TFLOP/s and their
fractions of the MI355X peaks) sit beside it.  `roofline` describes the
dominant kernel (the GEMM) from HIP events around every GEMM launch in the
timed steps.  `cpu_baseline` times the CPU oracle on the same step (all 8192
tokens by default; --cpu-sample-tokens bounds it).

`components.mxfp4` times the comparison format on the same tensors after the
NVFP4 step (not part of `value`): MXFP4 (32-element blocks, E8M0 scales, no
tensor scale, no Hadamard) row and column quantization of W, X (RNE) and dY
(SR), then the same three GEMMs on the block-scaled FP4 matrix instruction.
`components.linear_module` times the autograd layer (NVFP4Linear forward +
backward with BF16 outputs) against the same layer kept in BF16, and the
NVFP4 -> BF16 dequantization of W.  `components.hbm_copy_GBps` is the
achievable HBM rate measured live (an elementwise kernel reading and writing
1 GiB each), the reference for the quantize rates beside the 8 TB/s peak.
`components.quantize_sweep` times the quantize-only workload on its own
tensors (bf16 8192x5120 and 8192x20480, N(0,1) with 0.1% 100x outliers):
one row-1D nvfp4_quantize call each (tensor amax pass + cast pass), RNE and
SR, with the algorithmic bytes of the call (input once, codes, scales).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
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
MFMA_FP4_PEAK = 10100.0        # dense FP4 MFMA, TFLOP/s (context)

TOKENS, D_IN, D_OUT = 8192, 5120, 20480

# HBM bytes per k_gemm_nvfp4 launch (mean over the Fprop, Dgrad and Wgrad
# launches of this workload) from two rocprofv3 --pmc runs of
#   bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-probe-mib 1024
# FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (KiB -> bytes): the factors are what the
# same counters read for the 1 GiB read + 1 GiB write elementwise probe
# (FETCH_SIZE 512 MiB, WRITE_SIZE 1024 MiB).  Valid only for the kernel
# sources (gemm.hip + gemm_tiling.hpp) with this hash; any other source
# reports null.
GEMM_TRAFFIC = dict(src_sha256="d9aa8b7359bb0f9b8f22da021987d3b8164ca536f12b478f6a465e6b86a25ae1",
                    bytes_per_launch=1.1573e+09, fetch_bytes=7.0982e+08, write_bytes=4.4747e+08)
GEMM_SOURCES = ("gemm.hip", "gemm_tiling.hpp")


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
    p.add_argument("--cpu-sample-tokens", type=int, default=8192)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (calibrates "
                        "the FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    return p.parse_args()


def make_inputs():
    from bit_microscaled_quantized_amd import synth
    d = synth.ffn_up(TOKENS, D_IN, D_OUT)
    return dict(x=synth.f32_to_bf16_bits(d["x"]), w=synth.f32_to_bf16_bits(d["w"]),
                dy=synth.f32_to_bf16_bits(d["dy"]), sign_mask=d["sign_mask"],
                seed_row=d["sr_seed_row"], seed_col=d["sr_seed_col"])


def quantize_bytes():
    """Algorithmic bytes of the three quantize calls of a step: input read once,
    codes (0.5 B/elem) and scales (1/16 B/elem, 1/256 B/elem for 2D tiles)
    written; the 2D call also writes its transposed copy, the row + RHT calls
    write both a row-1D and an RHT column quantization."""
    T, I, O = TOKENS, D_IN, D_OUT
    w = O * I * 2 + 2 * (O * I // 2 + O * I // 256)
    x = T * I * 2 + 2 * (T * I // 2 + T * I // 16)
    dy = T * O * 2 + 2 * (T * O // 2 + T * O // 16)
    return dict(w=w, x=x, dy=dy)


def gpu_bench(inp, steps, warmup):
    import torch
    import bit_microscaled_quantized_amd as nv
    from bit_microscaled_quantized_amd.linear import LinearStep

    nv.load_library()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev)

    x, w, dy = up(inp["x"]), up(inp["w"]), up(inp["dy"])
    st = LinearStep(TOKENS, D_IN, D_OUT, device=dev)
    bf = nv.NVFP4_BF16
    T, I, O = TOKENS, D_IN, D_OUT
    mask, s_row, s_col = inp["sign_mask"], inp["seed_row"], inp["seed_col"]

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def one_step(rec):
        """One whole step; rec collects (name, start, end) events."""
        def timed(name, fn):
            if rec is None:
                fn()
                return
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            rec.append((name, a, b))
        # X first: its amax pass then follows the previous step's Wgrad GEMM
        # (non-temporal output) rather than the 2D cast's row-major stores
        qx, b_ = st.qx, st.qx_t
        timed("quant_x_row_rht", lambda: nv.nvfp4_quantize_row_rht(
            x, bf, T, I, I, nv.NVFP4_RNE, 0, qx.codes, qx.scales, qx.ts, qx.amax, mask,
            nv.NVFP4_RNE, 0, b_.codes, b_.scales, b_.ts, b_.amax))
        q = st.qw
        timed("quant_w_2d", lambda: nv.nvfp4_quantize(
            w, bf, O, I, I, nv.NVFP4_TILE_2D, nv.NVFP4_RNE, 0, q.codes, q.scales, q.codes_t,
            q.scales_t, q.ts, q.amax))
        timed("gemm_fprop", lambda: nv.nvfp4_gemm(
            T, O, I, qx.codes, qx.scales, qx.ts, q.codes, q.scales, 16, q.ts, st.y, O, 0.0, workspace=st.ws))
        qd, a_ = st.qdy, st.qdy_t
        timed("quant_dy_row_rht_sr", lambda: nv.nvfp4_quantize_row_rht(
            dy, bf, T, O, O, nv.NVFP4_SR, s_row, qd.codes, qd.scales, qd.ts, qd.amax, mask,
            nv.NVFP4_SR, s_col, a_.codes, a_.scales, a_.ts, a_.amax))
        timed("gemm_dgrad", lambda: nv.nvfp4_gemm(
            T, I, O, qd.codes, qd.scales, qd.ts, q.codes_t, q.scales_t, 16, q.ts, st.dx, I, 0.0, workspace=st.ws))
        timed("gemm_wgrad", lambda: nv.nvfp4_gemm(
            O, I, T, a_.codes, a_.scales, a_.ts, b_.codes, b_.scales, 1, b_.ts, st.dw, I, 0.0, workspace=st.ws))

    for _ in range(warmup):
        one_step(None)
    torch.cuda.synchronize()

    # whole-step wall time: K steps between two synchronizations, no events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step(None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-call HIP-event durations over another K steps on the same stream
    rec = []
    for _ in range(steps):
        one_step(rec)
    torch.cuda.synchronize()
    per = {}
    for name, a, b in rec:
        per.setdefault(name, []).append(a.elapsed_time(b))
    per = {k: float(np.mean(v)) for k, v in per.items()}
    mx = mx_bench(x, w, dy, s_row, s_col, steps, warmup)
    mod = module_bench(x, w, dy, st, steps, warmup)
    return wall / steps, per, mx, mod


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


def copy_bench(mib=1024, steps=10, warmup=3):
    """Achievable HBM rate on this GPU: an elementwise kernel (torch.neg) that
    reads and writes `mib` MiB each, read + write bytes per second (GB/s)."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = _events_ms(torch, lambda: torch.neg(src, out=dst), steps, warmup)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (mib << 20) / (ms * 1e-3) / 1e9


def module_bench(x, w, dy, st, steps, warmup):
    """The autograd layer on the same tensors: NVFP4Linear forward + backward
    (quantize, Fprop, Dgrad, Wgrad, BF16 outputs) against the same layer kept
    in BF16 (torch's BF16 matmul); and NVFP4 -> BF16 dequantization of W."""
    import torch
    import bit_microscaled_quantized_amd as nv
    from bit_microscaled_quantized_amd.module import NVFP4Linear
    T, I, O = TOKENS, D_IN, D_OUT
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
    q = st.qw  # W quantized by the NVFP4 step above
    wd = torch.empty((O, I), dtype=torch.bfloat16, device=x.device)
    ms = _events_ms(torch, lambda: nv.nvfp4_dequantize(q.codes, q.scales, 16, q.ts, O, I, nv.NVFP4_BF16,
                                                       wd, I), steps, warmup)
    nbytes = O * I // 2 + O * I // 256 + O * I * 2
    out["dequant_w_bf16_ms"] = round(ms, 4)
    out["dequant_w_bf16_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["dequant_frac_hbm"] = round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    return out


def mx_quantize_bytes():
    """Algorithmic bytes of each MXFP4 quantize call of the comparison step:
    bf16 input read once, codes (0.5 B/elem) and E8M0 scales (1/32 B/elem)
    written."""
    def one(n):
        return n * 2 + n // 2 + n // 32
    T, I, O = TOKENS, D_IN, D_OUT
    return dict(w_row=one(O * I), w_col=one(O * I), x_row=one(T * I), x_col=one(T * I),
                dy_row_sr=one(T * O), dy_col_sr=one(T * O))


def mx_bench(x, w, dy, s_row, s_col, steps, warmup):
    """The MXFP4 comparison step on the same device tensors: each of the six
    quantize calls and three GEMMs timed with HIP events on the current
    stream, averaged over `steps` steps after `warmup` untimed ones."""
    import torch
    import bit_microscaled_quantized_amd as nv
    dev = x.device
    T, I, O = TOKENS, D_IN, D_OUT
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
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    rec = []
    for _ in range(steps):
        for name, fn in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            rec.append((name, a, b))
    torch.cuda.synchronize()
    per = {}
    for name, a, b in rec:
        per.setdefault(name, []).append(a.elapsed_time(b))
    per = {k: float(np.mean(v)) for k, v in per.items()}
    qb = mx_quantize_bytes()
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


def sweep_bench(steps, warmup):
    """The quantize-only workload: each bf16 tensor quantized row-1D by one
    nvfp4_quantize call (zero amax, tensor amax pass, cast pass), RNE and SR,
    mean HIP-event time per call on the current stream.  GB/s counts the
    call's algorithmic bytes: the input read once (2 B/elem), codes
    (0.5 B/elem) and E4M3 scales (1/16 B/elem)."""
    import torch
    import bit_microscaled_quantized_amd as nv
    from bit_microscaled_quantized_amd import synth
    dev = torch.device("cuda", 0)
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {}
    for which in (0, 1):
        xb = synth.f32_to_bf16_bits(synth.quantize_sweep(which))
        R, C = xb.shape
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        codes, scales = torch.empty((R, C // 2), **u8), torch.empty((R, C // 16), **u8)
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        am = torch.empty(1, dtype=torch.float32, device=dev)
        nbytes = R * C * 2 + R * C // 2 + R * C // 16
        for rname, rnd, seed in (("rne", nv.NVFP4_RNE, 0), ("sr", nv.NVFP4_SR, 3)):
            ms = _events_ms(torch, lambda: nv.nvfp4_quantize(
                x, nv.NVFP4_BF16, R, C, C, nv.NVFP4_ROW_1D, rnd, seed, codes, scales, None, None,
                ts, am), steps, warmup)
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[f"{R}x{C}_{rname}"] = dict(ms=round(ms, 4), GBps=round(gbs, 1),
                                          frac_hbm=round(gbs / HBM_PEAK_GBS, 4), bytes=nbytes)
        del x, codes, scales
        torch.cuda.empty_cache()
    tot_b = sum(v["bytes"] for v in out.values())
    tot_ms = sum(v["ms"] for v in out.values())
    out["all"] = dict(GBps=round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
                      frac_hbm=round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    return out


def cpu_baseline(inp, tokens):
    """The oracle, as it stands, on the same step restricted to the first
    `tokens` tokens (full weight): five quantizations plus the three FP64
    contractions of its dequantized operands."""
    import oracle as ora
    from threadpoolctl import threadpool_info
    x, w, dy = inp["x"][:tokens], inp["w"], inp["dy"][:tokens]
    mask, s_row, s_col = inp["sign_mask"], inp["seed_row"], inp["seed_col"]
    t0 = time.perf_counter()
    qw = ora.quantize(w, ora.TILE_2D, ora.RNE)
    qx = ora.quantize(x, ora.ROW_1D, ora.RNE)
    y = ora.gemm_f64(ora.dequant(qx["codes"], qx["scales"], qx["tensor_scale"]),
                     ora.dequant(qw["codes"], qw["scales"], qw["tensor_scale"], 16))
    qd = ora.quantize(dy, ora.ROW_1D, ora.SR, s_row)
    dx = ora.gemm_f64(ora.dequant(qd["codes"], qd["scales"], qd["tensor_scale"]),
                      ora.dequant(qw["codes_t"], qw["scales_t"], qw["tensor_scale"], 16))
    qdt = ora.rht_quantize(dy, mask, ora.SR, s_col)
    qxt = ora.rht_quantize(x, mask, ora.RNE)
    dw = ora.gemm_f64(ora.dequant(qdt["codes"], qdt["scales"], qdt["tensor_scale"]),
                      ora.dequant(qxt["codes"], qxt["scales"], qxt["tensor_scale"]))
    dt = time.perf_counter() - t0
    del y, dx, dw
    flops = 3 * 2.0 * tokens * D_IN * D_OUT
    blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=max(ora.num_threads(), blas),
                kind="oracle", seconds=dt,
                sample=f"same step on the first {tokens} of {TOKENS} tokens with the full "
                       f"{D_OUT}x{D_IN} weight: W 2D, X row, dY row SR, RHT(dY) SR, RHT(X) "
                       f"quantization in the C oracle (OpenMP) + 3 FP64 BLAS contractions")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sharded path is a design, not built)", file=sys.stderr)
        sys.exit(2)
    inp = make_inputs()
    ms_step, per, mx, mod = gpu_bench(inp, args.steps, args.warmup)
    copy_gbs = copy_bench()
    sweep = sweep_bench(args.steps, args.warmup)
    if args.copy_probe_mib:
        import torch
        # an elementwise kernel (not a DMA copy, which no counter sees) that
        # reads and writes exactly n bytes
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    ms_step *= 1e3

    gemm_flops = 2.0 * TOKENS * D_IN * D_OUT  # each of the three GEMMs
    gemm_ms = np.mean([per["gemm_fprop"], per["gemm_dgrad"], per["gemm_wgrad"]])
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    qb = quantize_bytes()
    qnames = dict(w="quant_w_2d", x="quant_x_row_rht", dy="quant_dy_row_rht_sr")
    q_ms = sum(per[qnames[k]] for k in qb)
    q_gbs = sum(qb.values()) / (q_ms * 1e-3) / 1e9
    value = 3 * gemm_flops / (ms_step * 1e-3) / 1e12

    traffic = None
    if GEMM_TRAFFIC is not None and GEMM_TRAFFIC["src_sha256"] == gemm_src_sha():
        traffic = GEMM_TRAFFIC["bytes_per_launch"]

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
            "workload": "ffn_up_fwd_bwd: X bf16 8192x5120 N(0,1), W bf16 20480x5120 N(0,0.02^2), "
                        "dY bf16 8192x20480 N(0,1e-3^2); W 2D RNE (+transposed), X row RNE, "
                        "dY row SR, RHT+col (dY SR, X RNE); Fprop, Dgrad, Wgrad NVFP4 GEMMs",
            "tokens": TOKENS, "d_in": D_IN, "d_out": D_OUT,
        },
        "roofline": {
            "kernel": "k_gemm_nvfp4",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": MFMA_F16_PEAK,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / MFMA_F16_PEAK, 4),
            "traffic": traffic,
            "avg_launch_ms": round(float(gemm_ms), 4),
            "flops_per_launch": gemm_flops,
        },
        "components": {
            "quantize_GBps": round(q_gbs, 1),
            "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
            "hbm_copy_GBps": round(copy_gbs, 1),
            "quantize_frac_of_copy": round(q_gbs / copy_gbs, 4),
            "quantize_sweep": sweep,
            "gemm_TFLOPs": round(gemm_tflops, 2),
            "gemm_frac_mfma_f16": round(gemm_tflops / MFMA_F16_PEAK, 4),
            "gemm_frac_mfma_fp4": round(gemm_tflops / MFMA_FP4_PEAK, 4),
            "per_call_ms": {k: round(v, 4) for k, v in per.items()},
            "quantize_bytes": qb,
            "mxfp4": mx,
            "linear_module": mod,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
