"""GPU parity of the quantize entry points against the CPU oracle: codes,
block scales, tensor scale and amax must match bit for bit.

Shapes span several workgroup tiles and end in ragged tails (rows/cols that
are multiples of 16 but not of the kernels' 512/64/1024-element tiles)."""
import json
import os

import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(kind, shape, seed):
    if kind == "normal":
        x = synth.normal(seed, shape)
    elif kind == "outliers":
        x = synth.normal_with_outliers(seed, shape, frac=0.01)
    elif kind == "t3":
        x = synth.student_t(seed, shape)
    elif kind == "lognormal":
        x = synth.lognormal_signed(seed, shape)
    else:
        raise ValueError(kind)
    return x


def _same(g, o, keys):
    for k in keys:
        if isinstance(o[k], float):
            assert np.float32(g[k]).tobytes() == np.float32(o[k]).tobytes(), (k, g[k], o[k])
        else:
            assert np.array_equal(g[k], o[k]), f"{k}: {gpuio.first_diff(g[k], o[k])}"


KEYS = ("codes", "scales", "tensor_scale", "amax")

ROW_SHAPES = [(16, 16), (48, 80), (32, 8208), (272, 528)]


@pytest.mark.parametrize("shape", ROW_SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_row1d_parity(ora, shape, rnd, dtype):
    x = _inputs("outliers", shape, 21 + shape[0])
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    seed = 0x1234_5678_9ABC_DEF0
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
    o = ora.quantize(x, ora.ROW_1D, rnd, seed)
    _same(g, o, KEYS)


@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
def test_row1d_strided_input(ora, rnd):
    x = synth.f32_to_bf16_bits(_inputs("t3", (64, 400), 31))
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, 99, ld=464)
    o = ora.quantize(x, ora.ROW_1D, rnd, 99)
    _same(g, o, KEYS)


COL_SHAPES = [(16, 16), (528, 80), (1040, 144), (48, 1040)]


@pytest.mark.parametrize("shape", COL_SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_col1d_parity(ora, shape, rnd, dtype):
    x = _inputs("t3", shape, 41 + shape[1])
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    g = gpuio.gpu_quantize(x, nv.NVFP4_COL_1D, rnd, 7)
    o = ora.quantize(x, ora.COL_1D, rnd, 7)
    _same(g, o, KEYS)


TILE_SHAPES = [(16, 16), (80, 48), (208, 144), (64, 1040)]


@pytest.mark.parametrize("shape", TILE_SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tile2d_parity(ora, shape, rnd, dtype):
    x = _inputs("normal", shape, 51 + shape[0]) * np.float32(0.02)
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    g = gpuio.gpu_quantize(x, nv.NVFP4_TILE_2D, rnd, 3)
    o = ora.quantize(x, ora.TILE_2D, rnd, 3)
    _same(g, o, KEYS + ("codes_t", "scales_t"))


def test_tile2d_without_transpose(ora):
    x = synth.f32_to_bf16_bits(_inputs("normal", (96, 112), 57))
    g = gpuio.gpu_quantize(x, nv.NVFP4_TILE_2D, nv.NVFP4_RNE, 0, transpose=False)
    o = ora.quantize(x, ora.TILE_2D, ora.RNE, 0)
    _same(g, o, KEYS)


RHT_SHAPES = [(16, 16), (528, 80), (1024, 208), (2064, 48)]


@pytest.mark.parametrize("shape", RHT_SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rht_parity(ora, shape, rnd, dtype):
    x = _inputs("t3", shape, 61 + shape[0])
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    mask = synth.sign_mask16(shape[0])
    g = gpuio.gpu_rht_quantize(x, mask, rnd, 11)
    o = ora.rht_quantize(x, mask, rnd, 11)
    _same(g, o, KEYS)


@pytest.mark.parametrize("shape", RHT_SHAPES)
@pytest.mark.parametrize("rnds", [(nv.NVFP4_RNE, nv.NVFP4_RNE), (nv.NVFP4_SR, nv.NVFP4_SR),
                                  (nv.NVFP4_RNE, nv.NVFP4_SR)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_row_rht_parity(ora, shape, rnds, dtype):
    """The fused call equals the two separate calls bit for bit, and both
    equal the oracle."""
    x = _inputs("outliers", shape, 71 + shape[1])
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    mask = synth.sign_mask16(shape[1])
    row_rnd, rht_rnd = rnds
    g_row, g_rht = gpuio.gpu_quantize_row_rht(x, mask, row_rnd, 21, rht_rnd, 22)
    _same(g_row, gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, row_rnd, 21), KEYS)
    _same(g_rht, gpuio.gpu_rht_quantize(x, mask, rht_rnd, 22), KEYS)
    _same(g_row, ora.quantize(x, ora.ROW_1D, row_rnd, 21), KEYS)
    _same(g_rht, ora.rht_quantize(x, mask, rht_rnd, 22), KEYS)


# ------------------------------------------------------------------ edge cases
def test_golden_worked_example_on_gpu(ora):
    g_ = json.load(open(os.path.join(GOLDEN, "row1d_rne_two_blocks.json")))
    rows, cols = g_["shape"]
    x = np.zeros((rows, cols), np.float32)
    x[0] = [-0.0 if v == "-0" else float(v) for v in g_["input_row0_fp32"]]
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, nv.NVFP4_RNE)
    assert [f"{b:02X}" for b in g["codes"][0]] == g_["expected_codes_row0_hex"]
    assert [f"{b:02X}" for b in g["scales"][0]] == g_["expected_scales_row0_hex"]
    assert np.float32(g["tensor_scale"]).view(np.uint32) == int(g_["expected_tensor_scale_bits"], 16)
    assert not g["codes"][1:].any() and not g["scales"][1:].any()


def test_golden_flt_max_clamps_on_gpu(ora):
    """The hand-derived example where both FLT_MAX clamps of the scale rule
    act (S_enc, and r_b in the second block)."""
    g_ = json.load(open(os.path.join(GOLDEN, "row1d_flt_max_clamps.json")))
    rows, cols = g_["shape"]
    x = np.zeros((rows, cols), np.float32)
    x[0] = [float.fromhex(v) for v in g_["input_row0_fp32_hex"]]
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, nv.NVFP4_RNE)
    assert [f"{b:02X}" for b in g["codes"][0]] == g_["expected_codes_row0_hex"]
    assert [f"{b:02X}" for b in g["scales"][0]] == g_["expected_scales_row0_hex"]
    assert np.float32(g["tensor_scale"]).view(np.uint32) == int(g_["expected_tensor_scale_bits"], 16)
    assert np.float32(g["amax"]).view(np.uint32) == int(g_["expected_amax_bits"], 16)
    assert not g["codes"][1:].any() and not g["scales"][1:].any()


def _clamp_tensor():
    """The clamp example's row repeated over a 32 x 64 tensor (transposed in
    alternate 16-row bands, so column blocks see the clamps too)."""
    g_ = json.load(open(os.path.join(GOLDEN, "row1d_flt_max_clamps.json")))
    row = np.array([float.fromhex(v) for v in g_["input_row0_fp32_hex"]], np.float32)
    x = np.zeros((32, 64), np.float32)
    x[0, :32] = row
    x[5, 32:] = -row
    x[16:, 7] = row[:16]
    x[16:, 40] = row[16:]
    return x


def _edge_tensors():
    out = {}
    out["flt_max_clamps"] = _clamp_tensor()
    out["zeros"] = np.zeros((32, 64), np.float32)
    z = np.zeros((32, 64), np.float32)
    z[::3, ::5] = -0.0
    z[7, 9] = 1.0
    out["neg_zero_and_one"] = z
    rng = np.random.default_rng(5)
    out["denormal"] = (rng.standard_normal((32, 64)) * 1e-39).astype(np.float32)
    out["tiny"] = (rng.standard_normal((32, 64)) * 1e-33).astype(np.float32)
    out["huge"] = (rng.standard_normal((32, 64)) * 1e37).astype(np.float32)
    sp = np.zeros((32, 64), np.float32)
    sp[3, 17] = -5.0
    out["single_spike"] = sp
    ties = np.tile(np.array([6, -3, 1.5, 0.5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -6, 0, 4, 2, 5.5],
                            np.float32), (32, 4))
    out["ties"] = ties
    wide = np.exp(rng.uniform(-40, 40, (32, 64))).astype(np.float32) * np.sign(rng.standard_normal((32, 64))).astype(np.float32)
    out["wide_range"] = wide
    return out


EDGE = _edge_tensors()


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("layout", [nv.NVFP4_ROW_1D, nv.NVFP4_COL_1D, nv.NVFP4_TILE_2D])
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
def test_edge_cases(ora, name, layout, rnd):
    x = EDGE[name]
    g = gpuio.gpu_quantize(x, layout, rnd, 17)
    o = ora.quantize(x, layout, rnd, 17)
    keys = KEYS + (("codes_t", "scales_t") if layout == nv.NVFP4_TILE_2D else ())
    _same(g, o, keys)


def _edge_rht_input(name, dtype):
    x = EDGE[name]
    if name == "huge":
        x = x * np.float32(0.01)  # keep the 16-term butterflies finite
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


# bf16 input takes the kernels' folded transform (the 1/4 inside the block
# multiplier) unless S_enc < 2^-100, as for "huge" (amax ~1e35): both paths
# are covered here.
@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases_rht(ora, name, rnd, dtype):
    x = _edge_rht_input(name, dtype)
    g = gpuio.gpu_rht_quantize(x, 0x5A5A, rnd, 17)
    o = ora.rht_quantize(x, 0x5A5A, rnd, 17)
    _same(g, o, KEYS)


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases_row_rht(ora, name, dtype):
    x = _edge_rht_input(name, dtype)
    for rnd in (nv.NVFP4_SR, nv.NVFP4_RNE):
        g_row, g_rht = gpuio.gpu_quantize_row_rht(x, 0x5A5A, rnd, 31, rnd, 32)
        _same(g_row, ora.quantize(x, ora.ROW_1D, rnd, 31), KEYS)
        _same(g_rht, ora.rht_quantize(x, 0x5A5A, rnd, 32), KEYS)


@pytest.mark.parametrize("s_exp", [-110, -101, -100.5, -99.5, -99, 6, 86])
def test_rht_fold_boundary_bf16(ora, s_exp):
    """bf16 input whose RHT amax puts S_enc = 2688 / amax near 2^s_exp, on
    either side of 2^-100 where the kernels switch between the folded and the
    unfolded transform, with small entries that make subnormal products; the
    result must not depend on the path."""
    rng = np.random.default_rng(int(s_exp * 2) + 300)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    x[:, ::7] *= np.float32(2.0 ** -120)
    # the RHT amax of these 64 x 96 normals is about 4.4
    x = (x * np.float32(2688.0 * 2.0 ** -s_exp / 4.4)).astype(np.float32)
    xb = synth.f32_to_bf16_bits(x)
    for rnd in (nv.NVFP4_RNE, nv.NVFP4_SR):
        g = gpuio.gpu_rht_quantize(xb, 0x3C5A, rnd, 41)
        _same(g, ora.rht_quantize(xb, 0x3C5A, rnd, 41), KEYS)
        g_row, g_rht = gpuio.gpu_quantize_row_rht(xb, 0x3C5A, rnd, 42, rnd, 43)
        _same(g_row, ora.quantize(xb, ora.ROW_1D, rnd, 42), KEYS)
        _same(g_rht, ora.rht_quantize(xb, 0x3C5A, rnd, 43), KEYS)


def test_e2m1_conversion_sweep(ora):
    """FP32 values spread over [0, 6] (every 277th bit pattern) plus dense
    windows of +-2048 ulps around every E2M1 value and rounding midpoint go
    through the cast.  Each block holds a +-6 anchor, so amax_t = 6, S_enc =
    448, e_b = 0x7E, r_b = 1 and v = x: RNE and SR codes must equal the oracle."""
    pts = [0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0]
    parts = [np.arange(0, 0x40C00001, 277, dtype=np.int64)]
    for t in pts:
        b = int(np.float32(t).view(np.uint32))
        parts.append(np.arange(b - 2048, min(b + 2048, 0x40C00001), dtype=np.int64))
    vals = np.concatenate(parts).astype(np.uint32).view(np.float32)
    n_blocks = -(-len(vals) // 15)
    n_blocks = -(-n_blocks // 1024) * 1024
    probe = np.zeros(n_blocks * 15, np.float32)
    probe[: len(vals)] = vals
    x = np.empty((n_blocks, 16), np.float32)
    x[:, 0] = np.where(np.arange(n_blocks) % 2 == 0, 6.0, -6.0)
    x[:, 1:] = probe.reshape(n_blocks, 15)
    x[1::3, 1:] *= -1
    x = x.reshape(-1, 1024)
    for rnd in (nv.NVFP4_RNE, nv.NVFP4_SR):
        g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, 5)
        o = ora.quantize(x, ora.ROW_1D, rnd, 5)
        _same(g, o, KEYS)


def test_e2m1_conversion_exhaustive(ora):
    """Every FP32 bit pattern with |x| <= 6 (1.09e9 magnitudes; every third
    block negated) through the row cast, RNE and SR, against the oracle, in
    chunks of 4M blocks.  Each block holds a +-6 anchor and 15 test values, so
    amax_t = 6, S_enc = 448, e_b = 0x7E, r_b = 1 and the cast sees v = x."""
    top = int(np.float32(6.0).view(np.uint32)) + 1
    blocks = 1 << 22
    per = 15 * blocks
    for rnd in (nv.NVFP4_RNE, nv.NVFP4_SR):
        checked = 0
        for start in range(0, top, per):
            u = np.arange(start, min(start + per, top), dtype=np.uint32)
            checked += len(u)
            probe = np.zeros(per, np.float32)
            probe[: len(u)] = u.view(np.float32)
            x = np.empty((blocks, 16), np.float32)
            x[:, 0] = np.where(np.arange(blocks) % 2 == 0, 6.0, -6.0)
            x[:, 1:] = probe.reshape(blocks, 15)
            x[1::3, 1:] *= -1
            x = x.reshape(-1, 4096)
            seed = 17 + start
            g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
            o = ora.quantize(x, ora.ROW_1D, rnd, seed)
            _same(g, o, KEYS)
        assert checked == top


def test_sr_is_unbiased_on_gpu():
    """Mean of SR-dequantized values over many seeds approaches the input:
    each draw is within one grid step of x, so the mean of n draws lies within
    5 sigma <= 5 * step / (2 sqrt(n)) of x (plus the 2^-16 resolution bias)."""
    x = synth.normal(71, (16, 256))
    acc = np.zeros(x.shape, np.float64)
    n = 200
    for s in range(n):
        g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, nv.NVFP4_SR, s)
        codes = g["codes"]
        nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(x.shape)
        mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])[nib & 7] * np.where(nib & 8, -1.0, 1.0)
        unit = np.repeat(np.array([_e4m3(int(e)) for e in g["scales"].reshape(-1)]).reshape(16, 16),
                         16, axis=1) * g["tensor_scale"]
        acc += mag * unit
    mean = acc / n
    r = np.abs(x) / unit
    step = np.where(r >= 4, 2.0, np.where(r >= 2, 1.0, 0.5)) * unit
    err = np.abs(mean - x)
    assert (err <= 5 * step / (2 * np.sqrt(n)) + step * 2.0 ** -16).mean() > 0.999


def _e4m3(e):
    ex, m = (e >> 3) & 15, e & 7
    return m * 2.0 ** -9 if ex == 0 else (1 + m / 8) * 2.0 ** (ex - 7)


def test_amax_output_is_overwritten():
    """The library zero-fills amax itself: stale contents do not leak in."""
    torch = gpuio.torch_cuda()
    x = synth.f32_to_bf16_bits(synth.normal(3, (32, 32)))
    xd = gpuio.to_dev(x)
    codes = torch.empty((32, 16), dtype=torch.uint8, device="cuda")
    scales = torch.empty((32, 2), dtype=torch.uint8, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    am = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    nv.nvfp4_quantize(xd, nv.NVFP4_BF16, 32, 32, 32, nv.NVFP4_ROW_1D, nv.NVFP4_RNE, 0, codes,
                      scales, None, None, ts, am)
    torch.cuda.synchronize()
    assert float(am.item()) == float(np.abs(synth.bf16_bits_to_f32(x)).max())
