"""GPU parity at full size on EVERY output, not on samples: the first chunk of
the large-token stress layer (the headline workload) and the quantize-only
tensors, with the oracle run over whole tensors (C, OpenMP) and FP64 BLAS.

* W 5120x20480 log-normal, 2D tiles RNE with the transposed copy;
* X_in chunk 8192x20480 log-normal, row-1D RNE + RHT column RNE (one call);
* dY chunk 8192x5120 log-normal, row-1D SR + RHT column SR (one call);
* Fprop, Dgrad and Wgrad of that chunk: every output element, relative
  Frobenius error <= 1e-5 against the FP64 product of the oracle's own
  dequantized operands;
* quantize-only tensors (bf16 8192x5120, which takes the single pass, and
  8192x20480, two passes; N(0,1) with 0.1 % 100x outliers), RNE and SR;
* the FFN up-projection layer (X 8192x5120, W 20480x5120, dY 8192x20480):
  its five quantizations and three GEMMs;
* the Wgrad case (dY, X 8192x5120 Student-t(3), RHT + column-1D, dY SR):
  both quantizations and dW;
* the MXFP4 comparison step on the FFN up-projection tensors: six
  quantizations and three GEMMs.

Codes, scales, tensor scale and amax are compared bit for bit."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu
TOL = 1e-5
KEYS = ("codes", "scales", "tensor_scale", "amax")
T, I, O = 8192, 20480, 5120  # chunk tokens, d_in, d_out


def _same(g, o, keys=KEYS):
    for k in keys:
        if isinstance(o[k], float):
            assert np.float32(g[k]).tobytes() == np.float32(o[k]).tobytes(), (k, g[k], o[k])
        else:
            assert np.array_equal(g[k], o[k]), f"{k}: {gpuio.first_diff(g[k], o[k])}"


@pytest.fixture(scope="module")
def stress_chunk(ora):
    d = synth.ffn_down(T, O, I)  # the headline's generator, one chunk's worth of tokens
    x = synth.f32_to_bf16_bits(d["x_in"])
    w = synth.f32_to_bf16_bits(d["w"])
    dy = synth.f32_to_bf16_bits(d["dy"])
    mask, base = d["sign_mask"], d["sr_seed_base"]
    gw = gpuio.gpu_quantize(w, nv.NVFP4_TILE_2D)
    gx_row, gx_rht = gpuio.gpu_quantize_row_rht(x, mask, nv.NVFP4_RNE, 0, nv.NVFP4_RNE, 0)
    gd_row, gd_rht = gpuio.gpu_quantize_row_rht(dy, mask, nv.NVFP4_SR, base, nv.NVFP4_SR, base + 1)
    ow = ora.quantize(w, ora.TILE_2D, ora.RNE)
    ox_row, ox_rht = ora.quantize(x, ora.ROW_1D, ora.RNE), ora.rht_quantize(x, mask, ora.RNE)
    od_row = ora.quantize(dy, ora.ROW_1D, ora.SR, base)
    od_rht = ora.rht_quantize(dy, mask, ora.SR, base + 1)
    return dict(g=dict(w=gw, x_row=gx_row, x_rht=gx_rht, d_row=gd_row, d_rht=gd_rht),
                o=dict(w=ow, x_row=ox_row, x_rht=ox_rht, d_row=od_row, d_rht=od_rht))


def test_stress_chunk_quantize_every_code(stress_chunk):
    g, o = stress_chunk["g"], stress_chunk["o"]
    _same(g["w"], o["w"], KEYS + ("codes_t", "scales_t"))
    for k in ("x_row", "x_rht", "d_row", "d_rht"):
        _same(g[k], o[k])


def _gemm_check(ora, c, a_q, a_rowdiv, b_codes, b_scales, b_ts, b_rowdiv):
    ref = ora.gemm_f64(ora.dequant(a_q["codes"], a_q["scales"], a_q["tensor_scale"], a_rowdiv),
                       ora.dequant(b_codes, b_scales, b_ts, b_rowdiv))
    err = gpuio.rel_fro(c, ref)
    assert err <= TOL, err
    return ref


@pytest.mark.parametrize("which", ["fprop", "dgrad", "wgrad"])
def test_stress_chunk_gemm_every_output(ora, stress_chunk, which):
    g, o = stress_chunk["g"], stress_chunk["o"]
    if which == "fprop":  # Y = X W^T: 8192 x 5120, K = 20480
        c = gpuio.gpu_gemm(T, O, I, g["x_row"]["dev"], g["w"]["dev"], 16)
        _gemm_check(ora, c, o["x_row"], 1, o["w"]["codes"], o["w"]["scales"], o["w"]["tensor_scale"], 16)
    elif which == "dgrad":  # dX = dY W: 8192 x 20480, K = 5120
        bw = dict(codes=g["w"]["dev"]["codes_t"], scales=g["w"]["dev"]["scales_t"], ts=g["w"]["dev"]["ts"])
        c = gpuio.gpu_gemm(T, I, O, g["d_row"]["dev"], bw, 16)
        _gemm_check(ora, c, o["d_row"], 1, o["w"]["codes_t"], o["w"]["scales_t"],
                    o["w"]["tensor_scale"], 16)
    else:  # dW = RHT(dY)^T RHT(X): 5120 x 20480, K = 8192
        c = gpuio.gpu_gemm(O, I, T, g["d_rht"]["dev"], g["x_rht"]["dev"], 1)
        _gemm_check(ora, c, o["d_rht"], 1, o["x_rht"]["codes"], o["x_rht"]["scales"],
                    o["x_rht"]["tensor_scale"], 1)


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
def test_quantize_only_every_code(ora, which, rnd):
    x = synth.f32_to_bf16_bits(synth.quantize_sweep(which))
    seed = 4321 + which
    _same(gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed), ora.quantize(x, ora.ROW_1D, rnd, seed))


@pytest.fixture(scope="module")
def ffn_up_step(ora):
    """The FFN up-projection layer: X 8192x5120, W 20480x5120, dY 8192x20480."""
    d = synth.ffn_up()
    x = synth.f32_to_bf16_bits(d["x"])
    w = synth.f32_to_bf16_bits(d["w"])
    dy = synth.f32_to_bf16_bits(d["dy"])
    mask, sr, sc = d["sign_mask"], d["sr_seed_row"], d["sr_seed_col"]
    g = dict(w=gpuio.gpu_quantize(w, nv.NVFP4_TILE_2D))
    g["x_row"], g["x_rht"] = gpuio.gpu_quantize_row_rht(x, mask, nv.NVFP4_RNE, 0, nv.NVFP4_RNE, 0)
    g["d_row"], g["d_rht"] = gpuio.gpu_quantize_row_rht(dy, mask, nv.NVFP4_SR, sr, nv.NVFP4_SR, sc)
    o = dict(w=ora.quantize(w, ora.TILE_2D, ora.RNE), x_row=ora.quantize(x, ora.ROW_1D, ora.RNE),
             x_rht=ora.rht_quantize(x, mask, ora.RNE), d_row=ora.quantize(dy, ora.ROW_1D, ora.SR, sr),
             d_rht=ora.rht_quantize(dy, mask, ora.SR, sc))
    return dict(g=g, o=o, shape=(x.shape[0], x.shape[1], w.shape[0]))


def test_ffn_up_quantize_every_code(ffn_up_step):
    g, o = ffn_up_step["g"], ffn_up_step["o"]
    _same(g["w"], o["w"], KEYS + ("codes_t", "scales_t"))
    for k in ("x_row", "x_rht", "d_row", "d_rht"):
        _same(g[k], o[k])


@pytest.mark.parametrize("which", ["fprop", "dgrad", "wgrad"])
def test_ffn_up_gemm_every_output(ora, ffn_up_step, which):
    g, o = ffn_up_step["g"], ffn_up_step["o"]
    t, i, f = ffn_up_step["shape"]  # tokens, d_in (hidden), d_out (ffn)
    if which == "fprop":  # Y = X W^T: t x f, K = i
        c = gpuio.gpu_gemm(t, f, i, g["x_row"]["dev"], g["w"]["dev"], 16)
        _gemm_check(ora, c, o["x_row"], 1, o["w"]["codes"], o["w"]["scales"], o["w"]["tensor_scale"], 16)
    elif which == "dgrad":  # dX = dY W: t x i, K = f
        bw = dict(codes=g["w"]["dev"]["codes_t"], scales=g["w"]["dev"]["scales_t"], ts=g["w"]["dev"]["ts"])
        c = gpuio.gpu_gemm(t, i, f, g["d_row"]["dev"], bw, 16)
        _gemm_check(ora, c, o["d_row"], 1, o["w"]["codes_t"], o["w"]["scales_t"],
                    o["w"]["tensor_scale"], 16)
    else:  # dW = RHT(dY)^T RHT(X): f x i, K = t
        c = gpuio.gpu_gemm(f, i, t, g["d_rht"]["dev"], g["x_rht"]["dev"], 1)
        _gemm_check(ora, c, o["d_rht"], 1, o["x_rht"]["codes"], o["x_rht"]["scales"],
                    o["x_rht"]["tensor_scale"], 1)


def test_wgrad_case_every_output(ora):
    """dY, X bf16 8192x5120 Student-t(3); RHT + column-1D (dY SR, X RNE); dW = dY^T X."""
    d = synth.wgrad_rht()
    dy, x = synth.f32_to_bf16_bits(d["dy"]), synth.f32_to_bf16_bits(d["x"])
    mask, seed = d["sign_mask"], d["sr_seed"]
    gd, gx = gpuio.gpu_rht_quantize(dy, mask, nv.NVFP4_SR, seed), gpuio.gpu_rht_quantize(x, mask)
    od, ox = ora.rht_quantize(dy, mask, ora.SR, seed), ora.rht_quantize(x, mask)
    _same(gd, od)
    _same(gx, ox)
    t, c_ = dy.shape
    c = gpuio.gpu_gemm(c_, c_, t, gd["dev"], gx["dev"], 1)
    _gemm_check(ora, c, od, 1, ox["codes"], ox["scales"], ox["tensor_scale"], 1)


def test_mxfp4_ffn_up_every_output(ora):
    """The MXFP4 comparison step on the FFN up-projection tensors, as bench.py
    runs it: W, X and dY in row and column layouts (dY with SR), Fprop, Dgrad
    and Wgrad; every code and scale, every GEMM output."""
    d = synth.ffn_up()
    x = synth.f32_to_bf16_bits(d["x"])
    w = synth.f32_to_bf16_bits(d["w"])
    dy = synth.f32_to_bf16_bits(d["dy"])
    sr, sc = d["sr_seed_row"], d["sr_seed_col"]
    R, C = nv.NVFP4_ROW_1D, nv.NVFP4_COL_1D
    q = {}
    for name, t, layout, rnd, seed in (("w_r", w, R, 0, 0), ("w_c", w, C, 0, 0), ("x_r", x, R, 0, 0),
                                       ("x_c", x, C, 0, 0), ("d_r", dy, R, 1, sr), ("d_c", dy, C, 1, sc)):
        g = gpuio.gpu_mx_quantize(t, layout, rnd, seed)
        o = ora.mx_quantize(t, ora.ROW_1D if layout == R else ora.COL_1D, rnd, seed)
        assert np.array_equal(g["codes"], o["codes"]), f"{name} codes: {gpuio.first_diff(g['codes'], o['codes'])}"
        assert np.array_equal(g["scales"], o["scales"]), f"{name} scales"
        q[name] = (g, o)
    tok, hid = x.shape
    ffn = w.shape[0]
    for a, b, (M, N, K) in (("x_r", "w_r", (tok, ffn, hid)), ("d_r", "w_c", (tok, hid, ffn)),
                            ("d_c", "x_c", (ffn, hid, tok))):
        (ga, oa), (gb, ob) = q[a], q[b]
        c = gpuio.gpu_mx_gemm(M, N, K, ga["dev"], gb["dev"])
        ref = ora.gemm_f64(ora.mx_dequant(oa["codes"], oa["scales"]), ora.mx_dequant(ob["codes"], ob["scales"]))
        err = gpuio.rel_fro(c, ref)
        assert err <= TOL, (a, b, err)
