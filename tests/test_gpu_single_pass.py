"""GPU parity of the single-pass row-1D quantize (one read of the input, the
tensor amax exchanged between co-resident workgroups) against the oracle and
against the two-pass path: codes, scales, tensor scale and amax bit for bit.

* the quantize-only workload's 8192 x 5120 bf16 tensor (the 84 MB that fits
  on chip), whole tensor, RNE and SR;
* ragged small shapes in bf16 and FP32;
* the paths it must not take: strided rows and tensors beyond the on-chip
  capacity go through two passes (no single-pass launch counted);
* slot use across streams: two streams quantizing at once;
* the bounded wait, forced from the host: with a spin limit of zero the
  workgroups that arrive before the tensor amax is published give up and are
  counted, every kernel ends, the last workgroup to leave encodes their
  blocks from memory, so the output is still exact, and the next call on the
  same slot is exact too."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu

KEYS = ("codes", "scales", "tensor_scale", "amax")


def _same(g, o):
    for k in KEYS:
        if isinstance(o[k], float):
            assert np.float32(g[k]).tobytes() == np.float32(o[k]).tobytes(), (k, g[k], o[k])
        else:
            assert np.array_equal(g[k], o[k]), f"{k}: {gpuio.first_diff(g[k], o[k])}"


def _launches():
    return nv.nvfp4_single_pass_stats()


@pytest.fixture(autouse=True)
def _defaults():
    nv.nvfp4_set_quantize_passes(0)
    nv.nvfp4_set_sync_spin_limit(1 << 14)
    yield
    nv.nvfp4_set_quantize_passes(0)
    nv.nvfp4_set_sync_spin_limit(1 << 14)


@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
def test_single_pass_quantize_sweep_tensor(ora, rnd):
    """8192 x 5120 bf16, N(0,1) + 0.1% 100x outliers: the whole tensor."""
    x = synth.f32_to_bf16_bits(synth.quantize_sweep(0))
    seed = 4321
    n0, g0 = _launches()
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
    n1, g1 = _launches()
    assert n1 == n0 + 1 and g1 == g0, "the 84 MB tensor must take the single pass"
    _same(g, ora.quantize(x, ora.ROW_1D, rnd, seed))
    nv.nvfp4_set_quantize_passes(2)
    two = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
    assert _launches()[0] == n1
    _same(g, two)


SHAPES = [(16, 16), (48, 80), (32, 8208), (272, 528), (1040, 4112)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_pass_ragged(ora, shape, rnd, dtype):
    x = synth.lognormal_signed(300 + shape[0], shape)
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    n0, g0 = _launches()
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, 77)
    n1, g1 = _launches()
    assert n1 == n0 + 1 and g1 == g0
    _same(g, ora.quantize(x, ora.ROW_1D, rnd, 77))


def test_two_pass_where_single_pass_does_not_apply(ora):
    # strided rows
    x = synth.f32_to_bf16_bits(synth.normal(5, (64, 400)))
    n0, _ = _launches()
    g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, nv.NVFP4_SR, 9, ld=464)
    assert _launches()[0] == n0
    _same(g, ora.quantize(x, ora.ROW_1D, nv.NVFP4_SR, 9))
    # 8192 x 20480 bf16 (335 MB) is beyond the on-chip capacity
    torch = gpuio.torch_cuda()
    xb = torch.zeros((8192, 20480), dtype=torch.int16, device="cuda")
    codes = torch.empty((8192, 10240), dtype=torch.uint8, device="cuda")
    scales = torch.empty((8192, 1280), dtype=torch.uint8, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_quantize(xb, nv.NVFP4_BF16, 8192, 20480, 20480, nv.NVFP4_ROW_1D, nv.NVFP4_RNE, 0, codes,
                      scales, None, None, ts, am)
    torch.cuda.synchronize()
    assert _launches()[0] == n0
    assert float(am.item()) == 0.0 and float(ts.item()) == 1.0 and not codes.any().item()


def test_single_pass_on_two_streams(ora):
    """Two streams quantize different tensors without synchronizing in between:
    each stream has its own exchange slot."""
    torch = gpuio.torch_cuda()
    xs = [synth.f32_to_bf16_bits(synth.student_t(60 + i, (2048, 5120))) for i in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    devs = [gpuio.to_dev(x) for x in xs]
    torch.cuda.synchronize()
    g0 = _launches()[1]
    for rep in range(3):
        outs = []
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                u8 = dict(dtype=torch.uint8, device="cuda")
                o = dict(codes=torch.empty((2048, 2560), **u8), scales=torch.empty((2048, 320), **u8),
                         ts=torch.empty(1, dtype=torch.float32, device="cuda"),
                         am=torch.empty(1, dtype=torch.float32, device="cuda"))
                nv.nvfp4_quantize(devs[i], nv.NVFP4_BF16, 2048, 5120, 5120, nv.NVFP4_ROW_1D, nv.NVFP4_SR,
                                  11 + i, o["codes"], o["scales"], None, None, o["ts"], o["am"])
                outs.append(o)
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            ref = ora.quantize(xs[i], ora.ROW_1D, ora.SR, 11 + i)
            got = dict(codes=gpuio.host(o["codes"]), scales=gpuio.host(o["scales"]),
                       tensor_scale=float(o["ts"].item()), amax=float(o["am"].item()))
            _same(got, ref)
    assert _launches()[1] == g0


def test_forced_give_up_ends_and_recovers(ora):
    """Spin limit zero: workgroups that arrive before the amax is published give
    up and are counted; the last one to leave encodes their blocks from
    memory, so the outputs are exact anyway, and the next call on the same
    stream and slot (default limit) is exact and gives up nothing."""
    torch = gpuio.torch_cuda()
    x = synth.f32_to_bf16_bits(synth.quantize_sweep(0))
    for rnd, seed in ((nv.NVFP4_RNE, 0), (nv.NVFP4_SR, 8)):
        n0, g0 = _launches()
        nv.nvfp4_set_sync_spin_limit(0)
        g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
        torch.cuda.synchronize()
        n1, g1 = _launches()
        assert n1 == n0 + 1
        assert g1 > g0, "with no polling the early workgroups must give up"
        ref = ora.quantize(x, ora.ROW_1D, rnd, seed)
        _same(g, ref)
        nv.nvfp4_set_sync_spin_limit(1 << 14)
        g = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D, rnd, seed)
        n2, g2 = _launches()
        assert n2 == n1 + 1 and g2 == g1
        _same(g, ref)
