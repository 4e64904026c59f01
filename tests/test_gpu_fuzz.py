"""Seeded shape fuzz and an exhaustive sweep of the device's block-scale path.

* Shape fuzz: 48 random cases, rows and columns multiples of 16 from 16 to
  4096 (at most 2^22 elements each), over every quantize entry point and
  layout (row-1D, column-1D, 2D with its transposed copy, RHT column, fused
  row + RHT), RNE and SR, bf16 and FP32, and four value distributions; codes,
  scales, tensor scale and amax bit for bit against the oracle.
* Block-scale sweeps: every FP32 block maximum in [0, amax_t] (over 1.1e9
  values each) as its own 16-element block [amax_b, 0, ..., 0] of an FP32
  tensor whose amax is amax_t, for amax_t = 2688 (S_enc = 1) and 1792
  (S_enc = 1.5), so the device computes e_b = E4M3(RN(amax_b / 6) * S_enc)
  for every FP32 input of the division and a wide cover of the encoder's
  inputs up to the top code; the scale bytes are compared with the oracle's
  nearest-even search."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu

KEYS = ("codes", "scales", "tensor_scale", "amax")


def _same(g, o, keys=KEYS):
    for k in keys:
        if isinstance(o[k], float):
            assert np.float32(g[k]).tobytes() == np.float32(o[k]).tobytes(), (k, g[k], o[k])
        else:
            assert np.array_equal(g[k], o[k]), f"{k}: {gpuio.first_diff(g[k], o[k])}"


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    while len(out) < 48:
        rows = 16 * int(rng.integers(1, 257))
        cols = 16 * int(rng.integers(1, 257))
        if rows * cols > 1 << 22:
            continue
        kind = ["row", "col", "tile", "rht", "row_rht"][len(out) % 5]
        dist = ["normal", "outliers", "t3", "lognormal"][int(rng.integers(0, 4))]
        rnd = int(rng.integers(0, 2))
        dt = ["bf16", "f32"][int(rng.integers(0, 2))]
        out.append((len(out), rows, cols, kind, dist, rnd, dt))
    return out


def _input(i, rows, cols, dist, dt):
    seed = 1000 + i
    if dist == "normal":
        x = synth.normal(seed, (rows, cols))
    elif dist == "outliers":
        x = synth.normal_with_outliers(seed, (rows, cols), frac=0.01)
    elif dist == "t3":
        x = synth.student_t(seed, (rows, cols))
    else:
        x = synth.lognormal_signed(seed, (rows, cols))
    return synth.f32_to_bf16_bits(x) if dt == "bf16" else x


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-{c[3]}-{c[4]}-r{c[5]}-{c[6]}")
def test_shape_fuzz(ora, case):
    i, rows, cols, kind, dist, rnd, dt = case
    x = _input(i, rows, cols, dist, dt)
    seed, mask = 77 + i, synth.sign_mask16(i)
    if kind == "row":
        _same(gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed), ora.quantize(x, ora.ROW_1D, rnd, seed))
    elif kind == "col":
        _same(gpuio.gpu_quantize(x, nv.NVFP4_COL_1D, rnd, seed), ora.quantize(x, ora.COL_1D, rnd, seed))
    elif kind == "tile":
        _same(gpuio.gpu_quantize(x, nv.NVFP4_TILE_2D, rnd, seed), ora.quantize(x, ora.TILE_2D, rnd, seed),
              KEYS + ("codes_t", "scales_t"))
    elif kind == "rht":
        _same(gpuio.gpu_rht_quantize(x, mask, rnd, seed), ora.rht_quantize(x, mask, rnd, seed))
    else:
        g_row, g_rht = gpuio.gpu_quantize_row_rht(x, mask, rnd, seed, 1 - rnd, seed + 1)
        _same(g_row, ora.quantize(x, ora.ROW_1D, rnd, seed))
        _same(g_rht, ora.rht_quantize(x, mask, 1 - rnd, seed + 1))


@pytest.mark.parametrize("amax_t", [2688.0, 1792.0])
def test_block_scale_every_fp32_block_amax(ora, amax_t):
    """Every FP32 block maximum in [0, amax_t] in its own block; amax_t = 2688
    gives S_enc = 1 (e_b = E4M3(RN(amax_b / 6))) and 1792 gives S_enc = 1.5
    (e_b = E4M3(RN(RN(amax_b / 6) * 1.5))), so between them the scale codes
    of most FP32 inputs of the encoder up to 448 are seen."""
    torch = gpuio.torch_cuda()
    top = int(np.float32(amax_t).view(np.uint32))  # inclusive
    s_enc = np.float32(2688.0) / np.float32(amax_t)
    chunk = 1 << 26
    rows = chunk + 16  # the last 16 rows: one block holding amax_t, the rest zero
    x = torch.zeros((rows, 16), dtype=torch.float32, device="cuda")
    x[chunk, 0] = amax_t
    u8 = dict(dtype=torch.uint8, device="cuda")
    codes = torch.empty((rows, 8), **u8)
    scales = torch.empty((rows, 1), **u8)
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    checked = 0
    for start in range(0, top + 1, chunk):
        n = min(chunk, top + 1 - start)
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        bits[n:] = 0
        x[:chunk, 0] = bits.to(torch.int32).view(torch.float32)
        nv.nvfp4_quantize(x, nv.NVFP4_F32, rows, 16, 16, nv.NVFP4_ROW_1D, nv.NVFP4_RNE, 0, codes,
                          scales, None, None, ts, am)
        torch.cuda.synchronize()
        assert float(am.item()) == amax_t and np.float32(ts.item()) == np.float32(1.0) / s_enc
        got = scales[:n, 0].cpu().numpy()
        amax_b = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = ora.block_scale_array(amax_b, float(s_enc))
        assert np.array_equal(got, want), gpuio.first_diff(got, want)
        assert int(scales[chunk, 0].item()) == 0x7E  # amax_t / 6 * S_enc = 448: the top code
        checked += n
    assert checked == top + 1
