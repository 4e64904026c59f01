"""GPU parity of nvfp4_gemm against the oracle's FP64 contraction of its own
exactly dequantized operands: relative Frobenius error <= 1e-5.

The bound: every product of two dequantized NVFP4 values is exact in FP32, so
the only rounding is the FP32 accumulation (about sqrt(K/16) * 2^-24 relative
for blocked sums, ~1e-6 at K = 32768) and the final alpha multiply (2^-24)."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from bit_microscaled_quantized_amd.linear import LinearStep
from tests import gpuio

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _deq(ora, q, rowdiv=1, t=False):
    if t:
        return ora.dequant(q["codes_t"], q["scales_t"], q["tensor_scale"], rowdiv)
    return ora.dequant(q["codes"], q["scales"], q["tensor_scale"], rowdiv)


def test_tiny_linear_256(ora):
    """X, W fp32 256x256 N(0,1): X row-1D RNE, W 2D RNE, Y = X W^T."""
    x, w = synth.tiny_linear()
    gx = gpuio.gpu_quantize(x, nv.NVFP4_ROW_1D)
    gw = gpuio.gpu_quantize(w, nv.NVFP4_TILE_2D)
    ox = ora.quantize(x, ora.ROW_1D)
    ow = ora.quantize(w, ora.TILE_2D)
    assert np.array_equal(gx["codes"], ox["codes"]) and np.array_equal(gw["codes"], ow["codes"])
    y = gpuio.gpu_gemm(256, 256, 256, gx["dev"], gw["dev"], 16)
    ref = ora.gemm_f64(_deq(ora, ox), _deq(ora, ow, 16))
    assert gpuio.rel_fro(y, ref) <= TOL
    # the triple loop agrees with BLAS on this size
    assert np.allclose(ora.gemm_f64_loop(_deq(ora, ox), _deq(ora, ow, 16)), ref, rtol=1e-12, atol=1e-9)


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (272, 528, 320), (528, 16, 256), (16, 784, 1088),
                                   (1024, 768, 2048)])
@pytest.mark.parametrize("rowdiv", [1, 16])
def test_gemm_shapes(ora, M, N, K, rowdiv):
    a = synth.f32_to_bf16_bits(synth.student_t(81 + M, (M, K)))
    b = synth.f32_to_bf16_bits(synth.normal(82 + N, (N, K)))
    la = nv.NVFP4_ROW_1D
    lb = nv.NVFP4_ROW_1D if rowdiv == 1 else nv.NVFP4_TILE_2D
    ga, gb = gpuio.gpu_quantize(a, la), gpuio.gpu_quantize(b, lb, transpose=False)
    oa, ob = ora.quantize(a, la), ora.quantize(b, lb, want_transpose=False)
    assert np.array_equal(ga["codes"], oa["codes"]) and np.array_equal(gb["codes"], ob["codes"])
    c = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], rowdiv)
    ref = ora.gemm_f64(_deq(ora, oa), _deq(ora, ob, rowdiv))
    assert gpuio.rel_fro(c, ref) <= TOL, gpuio.rel_fro(c, ref)
    # entries far from zero are individually accurate as well
    big = np.abs(ref) > 0.1 * np.abs(ref).max()
    assert (np.abs(c - ref)[big] <= 1e-4 * np.abs(ref)[big]).all()


def test_gemm_beta_accumulates(ora):
    M, N, K = 272, 256, 192
    a = synth.normal(91, (M, K))
    b = synth.normal(92, (N, K))
    c0 = synth.normal(93, (M, N))
    ga, gb = gpuio.gpu_quantize(a, nv.NVFP4_ROW_1D), gpuio.gpu_quantize(b, nv.NVFP4_ROW_1D)
    oa, ob = ora.quantize(a, ora.ROW_1D), ora.quantize(b, ora.ROW_1D)
    c = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1, c0=c0, beta=1.0)
    ref = ora.gemm_f64(_deq(ora, oa), _deq(ora, ob), c0, 1.0)
    assert gpuio.rel_fro(c, ref) <= TOL


def test_gemm_zero_operand(ora):
    M = N = K = 256
    a = np.zeros((M, K), np.float32)
    b = synth.normal(94, (N, K))
    ga, gb = gpuio.gpu_quantize(a, nv.NVFP4_ROW_1D), gpuio.gpu_quantize(b, nv.NVFP4_ROW_1D)
    c = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1)
    assert not c.any()


def _operands(ora, M, N, K, seed):
    a = synth.f32_to_bf16_bits(synth.student_t(seed, (M, K)))
    b = synth.f32_to_bf16_bits(synth.normal(seed + 1, (N, K)))
    ga, gb = gpuio.gpu_quantize(a, nv.NVFP4_ROW_1D), gpuio.gpu_quantize(b, nv.NVFP4_ROW_1D)
    oa, ob = ora.quantize(a, ora.ROW_1D), ora.quantize(b, ora.ROW_1D)
    assert np.array_equal(ga["codes"], oa["codes"]) and np.array_equal(gb["codes"], ob["codes"])
    return ga, gb, ora.gemm_f64(_deq(ora, oa), _deq(ora, ob))


@pytest.mark.parametrize("M,N,K", [
    (512, 512, 4096),     # 4 tiles, all split (16 K stages)
    (272, 784, 2048),     # ragged 2 x 4 tiles, 8 stages per tile
    (4336, 4096, 4096),   # 17 x 16 = 272 tiles: one full round + a split tail
])
def test_gemm_split_tail(ora, M, N, K):
    """The split tail path (partial tiles in the workspace, ordered reduction)
    against the oracle, against the unsplit path, and run to run bit-identical."""
    ws = nv.nvfp4_gemm_workspace_size(M, N, K)
    assert ws > 0, "shape chosen to exercise the split"
    ga, gb, ref = _operands(ora, M, N, K, 111 + M)
    c1 = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1)
    c2 = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1)
    c0 = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1, workspace=None)
    small = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1, workspace=ws - 16)
    assert np.isfinite(c1).all()
    assert c1.tobytes() == c2.tobytes(), "split result not deterministic"
    assert c0.tobytes() == small.tobytes(), "too small a workspace must fall back to the unsplit path"
    for c in (c1, c0):
        assert gpuio.rel_fro(c, ref) <= TOL, gpuio.rel_fro(c, ref)


def test_gemm_split_tail_accumulates(ora):
    M, N, K = 512, 272, 4096
    ga, gb, ref = _operands(ora, M, N, K, 121)
    c0 = synth.normal(123, (M, N))
    assert nv.nvfp4_gemm_workspace_size(M, N, K) > 0
    c = gpuio.gpu_gemm(M, N, K, ga["dev"], gb["dev"], 1, c0=c0, beta=1.0)
    assert gpuio.rel_fro(c, ref + c0) <= TOL


def test_gemm_workspace_size_bounds():
    torch = gpuio.torch_cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, N, K in [(256, 256, 64), (8192, 20480, 5120), (8192, 5120, 20480), (20480, 5120, 8192),
                    (4096, 4096, 65536)]:
        ws = nv.nvfp4_gemm_workspace_size(M, N, K)
        assert 0 <= ws <= cus * 256 * 256 * 4
    assert nv.nvfp4_gemm_workspace_size(256, 256, 64) == 0  # a single short tile is not split


def test_linear_step_fprop_dgrad_wgrad(ora):
    """The whole recipe on a small layer with ragged tiles: T=384, IN=320,
    OUT=576; every quantized operand bit-exact, every GEMM within 1e-5."""
    torch = gpuio.torch_cuda()
    T, IN, OUT = 384, 320, 576
    x = synth.f32_to_bf16_bits(synth.normal(101, (T, IN)))
    w = synth.f32_to_bf16_bits(synth.normal(102, (OUT, IN), 0.02))
    dy = synth.f32_to_bf16_bits(synth.normal(103, (T, OUT), 1e-3))
    mask, s_row, s_col = synth.sign_mask16(104), 105, 106
    step = LinearStep(T, IN, OUT)
    xd, wd, dyd = gpuio.to_dev(x), gpuio.to_dev(w), gpuio.to_dev(dy)
    step.step(xd, wd, dyd, nv.NVFP4_BF16, mask, s_row, s_col)
    torch.cuda.synchronize()

    ox = ora.quantize(x, ora.ROW_1D)
    ow = ora.quantize(w, ora.TILE_2D)
    ody = ora.quantize(dy, ora.ROW_1D, ora.SR, s_row)
    ody_t = ora.rht_quantize(dy, mask, ora.SR, s_col)
    ox_t = ora.rht_quantize(x, mask, ora.RNE, 0)
    pairs = [(step.qx, ox, False), (step.qw, ow, True), (step.qdy, ody, False),
             (step.qdy_t, ody_t, False), (step.qx_t, ox_t, False)]
    for q, o, has_t in pairs:
        assert np.array_equal(gpuio.host(q.codes), o["codes"])
        assert np.array_equal(gpuio.host(q.scales), o["scales"])
        if has_t:
            assert np.array_equal(gpuio.host(q.codes_t), o["codes_t"])
            assert np.array_equal(gpuio.host(q.scales_t), o["scales_t"])

    y_ref = ora.gemm_f64(_deq(ora, ox), _deq(ora, ow, 16))
    dx_ref = ora.gemm_f64(_deq(ora, ody), _deq(ora, ow, 16, t=True))
    dw_ref = ora.gemm_f64(_deq(ora, ody_t), _deq(ora, ox_t))
    assert gpuio.rel_fro(gpuio.host(step.y), y_ref) <= TOL
    assert gpuio.rel_fro(gpuio.host(step.dx), dx_ref) <= TOL
    assert gpuio.rel_fro(gpuio.host(step.dw), dw_ref) <= TOL
    # the quantized weight is the same for forward and backward
    assert np.array_equal(_deq(ora, ow, 16).T, _deq(ora, ow, 16, t=True))
