"""Library calls captured in a HIP graph (torch.cuda.graph) and replayed.

A stream under capture cannot use the per-stream exchange slots (their epoch
is a host counter that a replay would not advance), so captured calls take
the slot-free forms: two passes, with each amax cleared by a small kernel and
reduced by per-workgroup atomics.  Those forms must give the same bytes as the
eager calls, which take the single passes and the slot-based amax reduction.

One graph holds, on bf16 inputs of single-pass size: a row-1D SR quantize, the
fused row + RHT call with RNE (a single pass when eager) and with SR, a 2D
weight quantize with its transposed copy, and an NVFP4 GEMM on the captured
outputs.  It is replayed three times, with eager library calls and
synchronizations between the replays and its outputs overwritten before each
one; every replay must reproduce the eager results bit for bit (codes, scales,
tensor scales, amaxes, GEMM output), and the eager results match the oracle.
No single-pass launch may be recorded by the capture."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu

T, C, O = 2048, 5120, 1024  # tokens, in features, out features


def _bufs(torch):
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    b = {}
    b["q_c"], b["q_s"] = torch.empty((T, C // 2), **u8), torch.empty((T, C // 16), **u8)
    for p in ("xr", "dr"):  # row copies of x and dy
        b[p + "_c"], b[p + "_s"] = torch.empty((T, C // 2), **u8), torch.empty((T, C // 16), **u8)
    for p in ("xh", "dh"):  # RHT column copies
        b[p + "_c"], b[p + "_s"] = torch.empty((C, T // 2), **u8), torch.empty((C, T // 16), **u8)
    b["w_c"], b["w_s"] = torch.empty((O, C // 2), **u8), torch.empty((O // 16, C // 16), **u8)
    b["wt_c"], b["wt_s"] = torch.empty((C, O // 2), **u8), torch.empty((C // 16, O // 16), **u8)
    for k in ("q", "xr", "dr", "xh", "dh", "w"):
        b[k + "_t"], b[k + "_a"] = torch.empty(1, **f32), torch.empty(1, **f32)
    b["y"] = torch.empty((T, O), **f32)
    b["ws"] = torch.empty(max(nv.nvfp4_gemm_workspace_size(T, O, C), 16), **u8)
    return b


def _calls(x, dy, w, b):
    bf = nv.NVFP4_BF16
    nv.nvfp4_quantize(x, bf, T, C, C, nv.NVFP4_ROW_1D, nv.NVFP4_SR, 91, b["q_c"], b["q_s"], None, None,
                      b["q_t"], b["q_a"])
    nv.nvfp4_quantize_row_rht(x, bf, T, C, C, nv.NVFP4_RNE, 0, b["xr_c"], b["xr_s"], b["xr_t"], b["xr_a"],
                              0x5AA5, nv.NVFP4_RNE, 0, b["xh_c"], b["xh_s"], b["xh_t"], b["xh_a"])
    nv.nvfp4_quantize_row_rht(dy, bf, T, C, C, nv.NVFP4_SR, 92, b["dr_c"], b["dr_s"], b["dr_t"], b["dr_a"],
                              0x5AA5, nv.NVFP4_SR, 93, b["dh_c"], b["dh_s"], b["dh_t"], b["dh_a"])
    nv.nvfp4_quantize(w, bf, O, C, C, nv.NVFP4_TILE_2D, nv.NVFP4_RNE, 0, b["w_c"], b["w_s"], b["wt_c"],
                      b["wt_s"], b["w_t"], b["w_a"])
    nv.nvfp4_gemm(T, O, C, b["xr_c"], b["xr_s"], b["xr_t"], b["w_c"], b["w_s"], 16, b["w_t"], b["y"], O, 0.0,
                  workspace=b["ws"])


def _host(b):
    return {k: gpuio.host(v) for k, v in b.items() if k != "ws"}


def _same_all(got, want, what):
    for k in want:
        assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), \
            f"{what}: {k} differs ({gpuio.first_diff(got[k], want[k])})"


def test_captured_calls_replay_exactly(ora):
    torch = gpuio.torch_cuda()
    xs = synth.f32_to_bf16_bits(synth.normal_with_outliers(501, (T, C)))
    dys = synth.f32_to_bf16_bits(synth.lognormal_signed(502, (T, C)))
    ws = synth.f32_to_bf16_bits(synth.normal(503, (O, C), 0.02))
    x, dy, w = gpuio.to_dev(xs), gpuio.to_dev(dys), gpuio.to_dev(ws)

    eager, graph = _bufs(torch), _bufs(torch)
    n0, _ = nv.nvfp4_single_pass_stats()
    _calls(x, dy, w, eager)
    torch.cuda.synchronize()
    n1, _ = nv.nvfp4_single_pass_stats()
    assert n1 == n0 + 2, "eager: the row-1D SR call and the RNE fused call take single passes"
    want = _host(eager)

    # the eager results against the oracle
    q = ora.quantize(xs, ora.ROW_1D, ora.SR, 91)
    assert np.array_equal(want["q_c"], q["codes"]) and np.array_equal(want["q_s"], q["scales"])
    xr, xh = ora.quantize(xs, ora.ROW_1D, ora.RNE, 0), ora.rht_quantize(xs, 0x5AA5, ora.RNE, 0)
    dr, dh = ora.quantize(dys, ora.ROW_1D, ora.SR, 92), ora.rht_quantize(dys, 0x5AA5, ora.SR, 93)
    for k, o in (("xr", xr), ("xh", xh), ("dr", dr), ("dh", dh)):
        assert np.array_equal(want[k + "_c"], o["codes"]) and np.array_equal(want[k + "_s"], o["scales"]), k
        assert np.float32(want[k + "_a"][0]) == np.float32(o["amax"]), k
    w2 = ora.quantize(ws, ora.TILE_2D, ora.RNE, 0)
    assert np.array_equal(want["w_c"], w2["codes"]) and np.array_equal(want["wt_c"], w2["codes_t"])

    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            _calls(x, dy, w, graph)
    torch.cuda.synchronize()
    assert nv.nvfp4_single_pass_stats()[0] == n1, "a captured call must not take a single pass"

    for rep in range(3):
        for k, v in graph.items():  # overwrite every output before the replay
            if k != "ws":
                v.fill_(0xA5 if v.dtype == torch.uint8 else 7.0)
        # eager library work between replays, on the same stream and slot
        _calls(x, dy, w, eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same_all(_host(graph), want, f"replay {rep}")
        _same_all(_host(eager), want, f"eager call before replay {rep}")
