"""More streams than exchange slots.

Each (device, stream) that runs a quantize call takes one of the library's 64
exchange slots for the life of the process; once they are all taken, calls on
further streams run the slot-free two-pass forms (amax cleared by a small
kernel, per-workgroup atomics).  This test creates 72 HIP streams and runs a
single-pass-sized row-1D SR quantize and the fused RNE call on each: the
first new stream still finds a free slot (earlier tests of the process use at
most torch's 32 pooled streams and the default one) and takes single passes,
no stream past the 64th does, and every output is the same as on the first
stream (whose results the single-pass tests check against the oracle).

It leaves the process's slots exhausted, so it is collected after every test
that needs a free slot (only the GEMM-only allocation-free test follows)."""
import ctypes
import os

import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu

T, C, N = 1024, 5120, 72


def test_calls_beyond_the_slot_count_take_the_slot_free_path():
    torch = gpuio.torch_cuda()
    nv.load_library()
    # the HIP runtime the library itself is linked against (already loaded)
    hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
    x = gpuio.to_dev(synth.f32_to_bf16_bits(synth.student_t(611, (T, C))))
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    streams, outs, taken = [], [], []
    try:
        for i in range(N):
            s = ctypes.c_void_p()
            assert hip.hipStreamCreate(ctypes.byref(s)) == 0
            streams.append(s)
            o = dict(qc=torch.empty((T, C // 2), **u8), qs=torch.empty((T, C // 16), **u8),
                     rc=torch.empty((T, C // 2), **u8), rs=torch.empty((T, C // 16), **u8),
                     hc=torch.empty((C, T // 2), **u8), hs=torch.empty((C, T // 16), **u8),
                     f=torch.empty(6, **f32))
            torch.cuda.synchronize()
            n0 = nv.nvfp4_single_pass_stats()[0]
            f = o["f"]
            nv.nvfp4_quantize(x, nv.NVFP4_BF16, T, C, C, nv.NVFP4_ROW_1D, nv.NVFP4_SR, 7, o["qc"], o["qs"],
                              None, None, f[0:1], f[1:2], stream=s.value)
            nv.nvfp4_quantize_row_rht(x, nv.NVFP4_BF16, T, C, C, nv.NVFP4_RNE, 0, o["rc"], o["rs"], f[2:3],
                                      f[3:4], 0x3C3C, nv.NVFP4_RNE, 0, o["hc"], o["hs"], f[4:5], f[5:6],
                                      stream=s.value)
            assert hip.hipStreamSynchronize(s) == 0
            taken.append(nv.nvfp4_single_pass_stats()[0] - n0)
            outs.append({k: gpuio.host(v) for k, v in o.items()})
    finally:
        torch.cuda.synchronize()
        for s in streams:
            hip.hipStreamDestroy(s)
    assert taken[0] == 2, taken
    assert all(t == 0 for t in taken[64:]), taken
    for i in range(1, N):
        for k in outs[0]:
            assert np.array_equal(outs[i][k].view(np.uint8), outs[0][k].view(np.uint8)), (i, k)
