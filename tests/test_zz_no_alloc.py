"""nvfp4_gemm_noalloc, the allocation-free GEMM entry point, against
nvfp4_gemm with a caller workspace: two calls in a row on one stream, the
second with a smaller problem (and beta = 1), both split over K in their last
round of tiles, so the second call reuses the static workspace the first one
filled.  The results must be identical bit for bit (same kernels, same split
plan) and within 1e-5 relative Frobenius error of the FP64 oracle product."""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu


def _operands(ora, M, N, K, seed):
    a = synth.f32_to_bf16_bits(synth.student_t(seed, (M, K)))
    b = synth.f32_to_bf16_bits(synth.normal(seed + 1, (N, K)))
    ga = gpuio.gpu_quantize(a, nv.NVFP4_ROW_1D, nv.NVFP4_RNE)
    gb = gpuio.gpu_quantize(b, nv.NVFP4_ROW_1D, nv.NVFP4_RNE)
    oa = ora.quantize(a, ora.ROW_1D, ora.RNE)
    ob = ora.quantize(b, ora.ROW_1D, ora.RNE)
    ref = ora.gemm_f64(ora.dequant(oa["codes"], oa["scales"], oa["tensor_scale"]),
                       ora.dequant(ob["codes"], ob["scales"], ob["tensor_scale"]))
    return ga["dev"], gb["dev"], ref


def test_gemm_noalloc_matches_workspace_gemm_twice(ora):
    torch = gpuio.torch_cuda()
    # 12 x 8 = 96 output tiles, K = 2048: the tail splits in two over K;
    # then 4 x 5 = 20 tiles, K = 4096: split in four, a smaller problem
    cases = [(3072, 2048, 2048, 0.0, 5), (1024, 1280, 4096, 1.0, 9)]
    for M, N, K, beta, seed in cases:
        assert nv.nvfp4_gemm_workspace_size(M, N, K) > 0, "the case must use the split workspace"
        a, b, ref = _operands(ora, M, N, K, seed)
        c0 = synth.normal(seed + 2, (M, N))
        want = gpuio.gpu_gemm(M, N, K, a, b, 1, c0=c0, beta=beta)
        c = gpuio.to_dev(c0)
        nv.nvfp4_gemm_noalloc(M, N, K, a["codes"], a["scales"], a["ts"], b["codes"], b["scales"], 1,
                              b["ts"], c, N, beta)
        torch.cuda.synchronize()
        got = gpuio.host(c)
        assert np.array_equal(got, want), gpuio.first_diff(got, want)
        full_ref = ref + (c0.astype(np.float64) if beta else 0.0)
        assert gpuio.rel_fro(got, full_ref) <= 1e-5
