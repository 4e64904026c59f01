"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (LinearStep), checked on sampled outputs the oracle computes one by one:

* quantize sweep: bf16 8192x5120 and 8192x20480, N(0,1) + 0.1% 100x outliers,
  row-1D with RNE and SR;
* Wgrad case: dY, X bf16 8192x5120 Student-t(3), RHT + column-1D (dY SR, X RNE),
  dW = dY^T X (5120x5120, K = 8192);
* FFN up-projection step: X 8192x5120, W 20480x5120, dY 8192x20480 -- every
  operand of Fprop, Dgrad and Wgrad and every GEMM output;
* FFN down-projection stress layer: X_in 32768x20480, W 5120x20480,
  dY 32768x5120 with log-normal magnitudes, four 8192-token chunks on one
  stream, W quantized once, Wgrad accumulated with beta = 1.

The oracle takes each tensor amax over the whole tensor and encodes only the
sampled lines (16 blocks of 16 lines per tensor dimension: first, last and
random middle ones; 6 token blocks per step); codes and scales are compared
bit for bit on those lines.  GEMM
references are FP64 products of the oracle's own dequantized lines, compared
with the GPU output on the sampled row x column blocks (relative Frobenius
error <= 1e-5)."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from bit_microscaled_quantized_amd.linear import LinearStep
from tests import gpuio

pytestmark = pytest.mark.gpu
TOL = 1e-5
W16 = 16


def _starts(n, count, seed):
    """Starts of `count` 16-line blocks: first, last and random middle ones."""
    rng = np.random.default_rng(seed)
    s = {0, n - W16}
    while len(s) < count:
        s.add(int(rng.integers(1, n // W16 - 1)) * W16)
    return sorted(s)


def _idx(starts):
    return np.concatenate([np.arange(s, s + W16) for s in starts])


def _host(t):
    return t.cpu().numpy()


class OracleLines:
    """Oracle codes/scales of selected 16-line blocks of one quantized tensor,
    gathered in block order (the same order as _idx(starts))."""

    def __init__(self, fn, starts, tile=False):
        self.codes, self.scales = [], []
        for s in starts:
            o = fn((s // W16, s // W16 + 1) if tile else (s, s + W16))
            self.codes.append(o["codes"][s:s + W16])
            self.scales.append(o["scales"][s // W16:s // W16 + 1] if tile else o["scales"][s:s + W16])
        self.ts, self.amax, self.last = o["tensor_scale"], o["amax"], o

    def deq(self, ora, tile=False):
        c = np.concatenate(self.codes)
        s = np.concatenate(self.scales)
        if tile:
            s = np.repeat(s, W16, axis=0)
        return ora.dequant(c, s, self.ts, 1)


def _check(g_codes, g_scales, g_ts, g_amax, lines: OracleLines, starts, tile=False):
    for i, s in enumerate(starts):
        gc = g_codes[s:s + W16]
        assert np.array_equal(gc, lines.codes[i]), f"codes {s}..{s + W16}: {gpuio.first_diff(gc, lines.codes[i])}"
        gs = g_scales[s // W16:s // W16 + 1] if tile else g_scales[s:s + W16]
        assert np.array_equal(gs, lines.scales[i]), f"scales of lines {s}..{s + W16}"
    assert np.float32(g_ts).tobytes() == np.float32(lines.ts).tobytes()
    assert np.float32(g_amax).tobytes() == np.float32(lines.amax).tobytes()


def _gemm_block(ora, got, A, B, rows, cols, prev=None):
    ref = ora.gemm_f64(A, B)
    if prev is not None:
        ref = ref + prev
    err = gpuio.rel_fro(got[np.ix_(rows, cols)], ref)
    assert err <= TOL, f"relative Frobenius error {err:.3e} on the sampled block"
    return ref


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
def test_quantize_sweep_fullsize(ora, which, rnd):
    x = synth.f32_to_bf16_bits(synth.quantize_sweep(which))
    seed = 1234 + which
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
    starts = _starts(x.shape[0], 16, which)
    lines = OracleLines(lambda ln: ora.quantize(x, ora.ROW_1D, rnd, seed, lines=ln), starts)
    _check(g["codes"], g["scales"], g["tensor_scale"], g["amax"], lines, starts)


def test_wgrad_rht_fullsize(ora):
    d = synth.wgrad_rht()
    dy, x = synth.f32_to_bf16_bits(d["dy"]), synth.f32_to_bf16_bits(d["x"])
    T, C = dy.shape
    mask, seed = d["sign_mask"], d["sr_seed"]
    gdy = gpuio.gpu_rht_quantize(dy, mask, nv.NVFP4_SR, seed)
    gx = gpuio.gpu_rht_quantize(x, mask, nv.NVFP4_RNE, 0)
    c = gpuio.gpu_gemm(C, C, T, gdy["dev"], gx["dev"], 1)
    rs, cs = _starts(C, 16, 1), _starts(C, 16, 2)
    ly = OracleLines(lambda ln: ora.rht_quantize(dy, mask, ora.SR, seed, lines=ln), rs)
    lx = OracleLines(lambda ln: ora.rht_quantize(x, mask, ora.RNE, 0, lines=ln), cs)
    _check(gdy["codes"], gdy["scales"], gdy["tensor_scale"], gdy["amax"], ly, rs)
    _check(gx["codes"], gx["scales"], gx["tensor_scale"], gx["amax"], lx, cs)
    _gemm_block(ora, c, ly.deq(ora), lx.deq(ora), _idx(rs), _idx(cs))


def _check_step(ora, st, x, w, dy, mask, s_row, s_col, ts_, ti, to, ow_full):
    """Bit-exact sampled operands of one LinearStep and sampled Fprop / Dgrad
    outputs; returns the oracle's Wgrad operand lines for the caller's check.
    ts_, ti, to: starts of sampled token / input-feature / output-feature blocks;
    ow_full: the oracle's full 2D quantization of W (for the transposed copy)."""
    lx = OracleLines(lambda ln: ora.quantize(x, ora.ROW_1D, ora.RNE, 0, lines=ln), ts_)
    _check(_host(st.qx.codes), _host(st.qx.scales), st.qx.ts.item(), st.qx.amax.item(), lx, ts_)
    ld = OracleLines(lambda ln: ora.quantize(dy, ora.ROW_1D, ora.SR, s_row, lines=ln), ts_)
    _check(_host(st.qdy.codes), _host(st.qdy.scales), st.qdy.ts.item(), st.qdy.amax.item(), ld, ts_)
    ldt = OracleLines(lambda ln: ora.rht_quantize(dy, mask, ora.SR, s_col, lines=ln), to)
    _check(_host(st.qdy_t.codes), _host(st.qdy_t.scales), st.qdy_t.ts.item(), st.qdy_t.amax.item(), ldt, to)
    lxt = OracleLines(lambda ln: ora.rht_quantize(x, mask, ora.RNE, 0, lines=ln), ti)
    _check(_host(st.qx_t.codes), _host(st.qx_t.scales), st.qx_t.ts.item(), st.qx_t.amax.item(), lxt, ti)
    # weight: row-major tile rows (output features) and the transposed copy
    # (input features), both from the oracle's one 2D quantization
    lw = OracleLines(lambda ln: ow_full, to, tile=True)
    _check(_host(st.qw.codes), _host(st.qw.scales), st.qw.ts.item(), st.qw.amax.item(), lw, to, tile=True)
    owt = dict(codes=ow_full["codes_t"], scales=ow_full["scales_t"], tensor_scale=ow_full["tensor_scale"],
               amax=ow_full["amax"])
    lwt = OracleLines(lambda ln: owt, ti, tile=True)
    _check(_host(st.qw.codes_t), _host(st.qw.scales_t), st.qw.ts.item(), st.qw.amax.item(), lwt, ti, tile=True)
    rows, cin, cout = _idx(ts_), _idx(ti), _idx(to)
    _gemm_block(ora, _host(st.y), lx.deq(ora), lw.deq(ora, tile=True), rows, cout)
    _gemm_block(ora, _host(st.dx), ld.deq(ora), lwt.deq(ora, tile=True), rows, cin)
    return ldt, lxt


def test_ffn_up_step_fullsize(ora):
    torch = gpuio.torch_cuda()
    d = synth.ffn_up()
    x, w, dy = (synth.f32_to_bf16_bits(d[k]) for k in ("x", "w", "dy"))
    T, IN = x.shape
    OUT = w.shape[0]
    st = LinearStep(T, IN, OUT)
    mask, s_row, s_col = d["sign_mask"], d["sr_seed_row"], d["sr_seed_col"]
    st.step(gpuio.to_dev(x), gpuio.to_dev(w), gpuio.to_dev(dy), nv.NVFP4_BF16, mask, s_row, s_col)
    torch.cuda.synchronize()
    ow = ora.quantize(w, ora.TILE_2D, ora.RNE)
    ts_, ti, to = _starts(T, 6, 3), _starts(IN, 16, 4), _starts(OUT, 16, 5)
    ldt, lxt = _check_step(ora, st, x, w, dy, mask, s_row, s_col, ts_, ti, to, ow)
    _gemm_block(ora, _host(st.dw), ldt.deq(ora), lxt.deq(ora), _idx(to), _idx(ti))


def test_ffn_down_stress_chunked(ora):
    """Four 8192-token chunks through one LinearStep on one stream; W is
    quantized once and reused; Wgrad accumulates (beta = 1) into one dW."""
    torch = gpuio.torch_cuda()
    d = synth.ffn_down()
    x_in = synth.f32_to_bf16_bits(d["x_in"])
    w = synth.f32_to_bf16_bits(d["w"])
    dy = synth.f32_to_bf16_bits(d["dy"])
    mask, base = d["sign_mask"], d["sr_seed_base"]
    del d
    T_all, IN = x_in.shape
    OUT = w.shape[0]
    T = T_all // 4
    st = LinearStep(T, IN, OUT)
    st.quantize_weight(gpuio.to_dev(w), nv.NVFP4_BF16)
    ow = ora.quantize(w, ora.TILE_2D, ora.RNE)
    ts_, ti, to = _starts(T, 6, 6), _starts(IN, 16, 7), _starts(OUT, 16, 8)
    dw_ref = None
    for ch in range(4):
        xs = np.ascontiguousarray(x_in[ch * T:(ch + 1) * T])
        dys = np.ascontiguousarray(dy[ch * T:(ch + 1) * T])
        s_row, s_col = base + 2 * ch, base + 2 * ch + 1
        xd, dyd = gpuio.to_dev(xs), gpuio.to_dev(dys)
        st.forward(xd, nv.NVFP4_BF16)
        st.backward(xd, dyd, nv.NVFP4_BF16, mask, s_row, s_col, accumulate_wgrad=ch > 0)
        torch.cuda.synchronize()
        ldt, lxt = _check_step(ora, st, xs, w, dys, mask, s_row, s_col, ts_, ti, to, ow)
        part = ora.gemm_f64(ldt.deq(ora), lxt.deq(ora))
        dw_ref = part if dw_ref is None else dw_ref + part
        del xd, dyd
    err = gpuio.rel_fro(_host(st.dw)[np.ix_(_idx(to), _idx(ti))], dw_ref)
    assert err <= TOL, f"accumulated dW relative Frobenius error {err:.3e}"
