"""GPU parity of the MXFP4 entry points (the comparison format) against the
oracle: quantized codes and E8M0 scales bit for bit; GEMM outputs within 1e-5
relative Frobenius of the FP64 product of the oracle's exactly dequantized
operands (the block-scaled FP4 matrix instruction forms every product exactly
and sums in FP32)."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu
TOL = 1e-5

ROW_SHAPES = [(16, 32), (48, 96), (32, 8224), (272, 544)]
COL_SHAPES = [(32, 16), (544, 80), (1024, 208), (2080, 48)]


def _x(seed, shape, dtype):
    x = synth.normal_with_outliers(seed, shape, frac=0.01) * np.float32(np.exp((seed % 7) - 3))
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _same(g, o):
    assert np.array_equal(g["scales"], o["scales"]), gpuio.first_diff(g["scales"], o["scales"])
    assert np.array_equal(g["codes"], o["codes"]), gpuio.first_diff(g["codes"], o["codes"])


@pytest.mark.parametrize("shape", ROW_SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_row_parity(ora, shape, rnd, dtype):
    x = _x(201 + shape[1], shape, dtype)
    _same(gpuio.gpu_mx_quantize(x, nv.NVFP4_ROW_1D, rnd, 41), ora.mx_quantize(x, ora.ROW_1D, rnd, 41))


@pytest.mark.parametrize("shape", COL_SHAPES)
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_col_parity(ora, shape, rnd, dtype):
    x = _x(301 + shape[0], shape, dtype)
    _same(gpuio.gpu_mx_quantize(x, nv.NVFP4_COL_1D, rnd, 42), ora.mx_quantize(x, ora.COL_1D, rnd, 42))


def _edge():
    rng = np.random.default_rng(9)
    out = {"zeros": np.zeros((32, 64), np.float32)}
    z = np.zeros((32, 64), np.float32)
    z[3, 5] = -0.0
    z[7, 40] = 7.5        # saturates to 6 (scale 2^0)
    z[8, 33] = 2.0 ** -130  # block max in the subnormal range: scale clamped to 2^-127
    out["sparse"] = z
    out["denormal"] = (rng.standard_normal((32, 64)) * 1e-39).astype(np.float32)
    out["huge"] = (rng.standard_normal((32, 64)) * 1e37).astype(np.float32)
    ties = np.tile(np.array([6, -3, 1.5, 0.5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -6, 0, 4, 2, 5.5],
                            np.float32), (32, 4))
    out["ties"] = ties
    out["wide"] = (np.exp(rng.uniform(-40, 40, (32, 64))) * np.sign(rng.standard_normal((32, 64)))).astype(np.float32)
    return out


EDGE = _edge()


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("layout", [nv.NVFP4_ROW_1D, nv.NVFP4_COL_1D])
@pytest.mark.parametrize("rnd", [nv.NVFP4_RNE, nv.NVFP4_SR])
def test_mx_edge_cases(ora, name, layout, rnd):
    x = EDGE[name]
    _same(gpuio.gpu_mx_quantize(x, layout, rnd, 43), ora.mx_quantize(x, layout, rnd, 43))


def _operands(ora, M, N, K, seed):
    a = synth.f32_to_bf16_bits(synth.student_t(seed, (M, K)))
    b = synth.f32_to_bf16_bits(synth.normal(seed + 1, (N, K)))
    ga, gb = gpuio.gpu_mx_quantize(a, nv.NVFP4_ROW_1D), gpuio.gpu_mx_quantize(b, nv.NVFP4_ROW_1D)
    oa, ob = ora.mx_quantize(a, ora.ROW_1D), ora.mx_quantize(b, ora.ROW_1D)
    _same(ga, oa)
    _same(gb, ob)
    ref = ora.gemm_f64(ora.mx_dequant(oa["codes"], oa["scales"]), ora.mx_dequant(ob["codes"], ob["scales"]))
    return ga["dev"], gb["dev"], ref


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (272, 528, 384), (528, 16, 256), (16, 784, 1152),
                                   (1024, 768, 2048), (512, 512, 4096), (4336, 4096, 1024)])
def test_mx_gemm_shapes(ora, M, N, K):
    a, b, ref = _operands(ora, M, N, K, 401 + M)
    c = gpuio.gpu_mx_gemm(M, N, K, a, b)
    assert np.isfinite(c).all()
    assert gpuio.rel_fro(c, ref) <= TOL, gpuio.rel_fro(c, ref)
    c0 = gpuio.gpu_mx_gemm(M, N, K, a, b, workspace=None)
    assert gpuio.rel_fro(c0, ref) <= TOL


def test_mx_gemm_beta_accumulates(ora):
    M, N, K = 272, 256, 640
    a, b, ref = _operands(ora, M, N, K, 411)
    c0 = synth.normal(412, (M, N))
    c = gpuio.gpu_mx_gemm(M, N, K, a, b, c0=c0, beta=1.0)
    assert gpuio.rel_fro(c, ref + c0) <= TOL
