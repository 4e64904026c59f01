"""GPU parity of the working-precision pieces around the NVFP4 path and of the
autograd layer built from them:

* nvfp4_dequantize: oracle-made codes and scales (row-1D, 2D tile grid and
  its transposed copy, random bytes) uploaded to the GPU; FP32 and BF16
  outputs compared bit for bit with the oracle's dequant_f32 / dequant_bf16;
* nvfp4_gemm_bf16: oracle-quantized operands; each BF16 output within one
  BF16 rounding of the oracle's FP64 product (plus the FP32-accumulation
  tolerance of the FP32 GEMM), beta = 1 included;
* NVFP4Linear forward and backward against the oracle's recipe (X row RNE,
  W 2D RNE, dY row SR and RHT column SR, X RHT column RNE, with the layer's
  own sign mask and seeds), in BF16 and FP32, 2D and 3D inputs.
"""
import numpy as np
import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import synth
from tests import gpuio

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8   # one BF16 rounding (2^-9) with margin
TOL = 1e-5             # FP32-accumulated GEMM against the FP64 product


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _close_bf16(got_bits: np.ndarray, ref: np.ndarray, what: str):
    """Each BF16 output within one BF16 rounding of the FP64 reference, up to
    the FP32-accumulation error of the sum (bounded by TOL of its scale)."""
    got = _bf16_to_f32(got_bits).astype(np.float64)
    scale = np.sqrt(np.mean(ref ** 2)) + 1e-300
    bad = np.abs(got - ref) > BF16_REL * np.abs(ref) + TOL * scale
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs off, first at {np.argwhere(bad)[0]}"


# --- dequantize ---------------------------------------------------------------

@pytest.mark.parametrize("out_dt", [nv.NVFP4_F32, nv.NVFP4_BF16])
@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 272), (512, 1024), (272, 48)])
def test_dequantize_random_bytes(ora, out_dt, rows, cols):
    torch = gpuio.torch_cuda()
    rng = np.random.default_rng(rows * 7 + cols + out_dt)
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 127, (rows, cols // 16), dtype=np.uint8)
    for ts in (1.0, float(np.float32(3.7e-4)), float(np.float32(2.0 ** -128)), float(np.float32(5e30))):
        dts = torch.tensor([ts], dtype=torch.float32, device="cuda")
        ld = cols + 16
        out = torch.full((rows, ld), -1.0, dtype=torch.float32 if out_dt == nv.NVFP4_F32 else torch.bfloat16,
                         device="cuda")
        nv.nvfp4_dequantize(gpuio.to_dev(codes), gpuio.to_dev(scales), 1, dts, rows, cols, out_dt, out, ld)
        torch.cuda.synchronize()
        got = out.cpu()
        if out_dt == nv.NVFP4_F32:
            want = ora.dequant_f32(codes, scales, ts, 1)
            g = got.numpy()
            assert np.array_equal(g[:, :cols].view(np.uint32), want.view(np.uint32)), ts
            assert np.all(g[:, cols:] == -1.0)  # padding untouched
        else:
            want = ora.dequant_bf16(codes, scales, ts, 1)
            g = got.view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(g[:, :cols], want), ts
            assert np.all(g[:, cols:] == 0xBF80)


@pytest.mark.parametrize("out_dt", [nv.NVFP4_F32, nv.NVFP4_BF16])
def test_dequantize_2d_and_transposed(ora, out_dt):
    """A 2D quantization (oracle) dequantized on the GPU in both stored
    orientations; the transposed copy dequantizes to the transpose."""
    torch = gpuio.torch_cuda()
    w = synth.f32_to_bf16_bits(synth.normal(61, (320, 192)) * 0.02)
    q = ora.quantize(w, ora.TILE_2D, ora.RNE)
    ts = q["tensor_scale"]
    dts = torch.tensor([ts], dtype=torch.float32, device="cuda")
    tdt = torch.float32 if out_dt == nv.NVFP4_F32 else torch.bfloat16
    for codes, scales, (r, c) in ((q["codes"], q["scales"], (320, 192)), (q["codes_t"], q["scales_t"], (192, 320))):
        gd = gpuio.Guarded()
        out = gd.alloc((r, c), tdt)
        nv.nvfp4_dequantize(gpuio.to_dev(codes), gpuio.to_dev(scales), 16, dts, r, c, out_dt, out, c)
        torch.cuda.synchronize()
        gd.check()
        if out_dt == nv.NVFP4_F32:
            assert np.array_equal(out.cpu().numpy(), ora.dequant_f32(codes, scales, ts, 16))
        else:
            assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16),
                                  ora.dequant_bf16(codes, scales, ts, 16))
    d = ora.dequant_f32(q["codes"], q["scales"], ts, 16)
    dt_ = ora.dequant_f32(q["codes_t"], q["scales_t"], ts, 16)
    assert np.array_equal(d.T, dt_)


# --- BF16 GEMM output -----------------------------------------------------------

def _oracle_operands(ora, M, N, K, seed):
    a = synth.f32_to_bf16_bits(synth.normal(seed, (M, K)))
    b = synth.f32_to_bf16_bits(synth.normal(seed + 1, (N, K)) * 0.05)
    qa = ora.quantize(a, ora.ROW_1D, ora.RNE)
    qb = ora.quantize(b, ora.TILE_2D, ora.RNE)
    return qa, qb


def _dev_q(torch, q, codes="codes", scales="scales"):
    return dict(codes=gpuio.to_dev(q[codes]), scales=gpuio.to_dev(q[scales]),
                ts=torch.tensor([q["tensor_scale"]], dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (272, 528, 384), (1024, 768, 2048), (4352, 4096, 1024)])
def test_gemm_bf16_output(ora, M, N, K):
    torch = gpuio.torch_cuda()
    qa, qb = _oracle_operands(ora, M, N, K, M + N + K)
    da, db = _dev_q(torch, qa), _dev_q(torch, qb)
    ref = ora.gemm_f64(ora.dequant(qa["codes"], qa["scales"], qa["tensor_scale"]),
                       ora.dequant(qb["codes"], qb["scales"], qb["tensor_scale"], 16))
    gd = gpuio.Guarded()
    c = gd.alloc((M, N), torch.bfloat16)
    ws = gd.alloc((max(nv.nvfp4_gemm_workspace_size(M, N, K), 16),), torch.uint8)
    nv.nvfp4_gemm_bf16(M, N, K, da["codes"], da["scales"], da["ts"], db["codes"], db["scales"], 16,
                       db["ts"], c, N, 0.0, workspace=ws)
    torch.cuda.synchronize()
    gd.check()
    _close_bf16(c.cpu().view(torch.int16).numpy().view(np.uint16), ref, f"{M}x{N}x{K}")

    # beta = 1: the BF16 values already in C are widened, added in FP32, rounded once
    c0 = synth.f32_to_bf16_bits(synth.normal(7, (M, N)))
    cd = gpuio.to_dev(c0).view(torch.bfloat16)
    nv.nvfp4_gemm_bf16(M, N, K, da["codes"], da["scales"], da["ts"], db["codes"], db["scales"], 16,
                       db["ts"], cd, N, 1.0, workspace=ws)
    torch.cuda.synchronize()
    _close_bf16(cd.cpu().view(torch.int16).numpy().view(np.uint16), ref + _bf16_to_f32(c0), "beta=1")


# --- the autograd layer -------------------------------------------------------------

def _oracle_step(ora, x, w, dy, mask, s_row, s_col):
    qx = ora.quantize(x, ora.ROW_1D, ora.RNE)
    qw = ora.quantize(w, ora.TILE_2D, ora.RNE)
    y = ora.gemm_f64(ora.dequant(qx["codes"], qx["scales"], qx["tensor_scale"]),
                     ora.dequant(qw["codes"], qw["scales"], qw["tensor_scale"], 16))
    qd = ora.quantize(dy, ora.ROW_1D, ora.SR, s_row)
    dx = ora.gemm_f64(ora.dequant(qd["codes"], qd["scales"], qd["tensor_scale"]),
                      ora.dequant(qw["codes_t"], qw["scales_t"], qw["tensor_scale"], 16))
    qdt = ora.rht_quantize(dy, mask, ora.SR, s_col)
    qxt = ora.rht_quantize(x, mask, ora.RNE)
    dw = ora.gemm_f64(ora.dequant(qdt["codes"], qdt["scales"], qdt["tensor_scale"]),
                      ora.dequant(qxt["codes"], qxt["scales"], qxt["tensor_scale"]))
    return y, dx, dw


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,IN,OUT,batch", [(256, 192, 320, None), (512, 1024, 768, None), (2, 256, 128, 128)])
def test_nvfp4_linear_forward_backward(ora, dtype, T, IN, OUT, batch):
    torch = gpuio.torch_cuda()
    from bit_microscaled_quantized_amd.module import NVFP4Linear
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tokens = T * batch if batch else T
    layer = NVFP4Linear(IN, OUT, seed=T + IN + OUT, dtype=tdt)
    x32 = synth.normal(71 + T, (tokens, IN))
    dy32 = synth.normal(72 + T, (tokens, OUT)) * 1e-3
    if dtype == "bf16":
        x_h, dy_h = synth.f32_to_bf16_bits(x32), synth.f32_to_bf16_bits(dy32)
        w_h = layer.weight.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()
        xd = gpuio.to_dev(x_h).view(torch.bfloat16)
        dyd = gpuio.to_dev(dy_h).view(torch.bfloat16)
    else:
        x_h, dy_h = x32, dy32
        w_h = layer.weight.detach().cpu().numpy().copy()
        xd, dyd = gpuio.to_dev(x_h), gpuio.to_dev(dy_h)
    s_row = layer.seed_base + 2 * layer.calls
    if batch:
        xd = xd.reshape(batch, T, IN)
        dyd = dyd.reshape(batch, T, OUT)
    xd.requires_grad_(True)
    y = layer(xd)
    y.backward(dyd)
    torch.cuda.synchronize()
    assert y.dtype == tdt and y.shape == (*xd.shape[:-1], OUT)
    assert xd.grad.shape == xd.shape and layer.weight.grad.shape == layer.weight.shape
    ref_y, ref_dx, ref_dw = _oracle_step(ora, x_h, w_h, dy_h, layer.sign_mask, s_row, s_row + 1)
    outs = [(y.detach().reshape(tokens, OUT), ref_y, "y"), (xd.grad.reshape(tokens, IN), ref_dx, "dx"),
            (layer.weight.grad, ref_dw, "dw")]
    for got, ref, what in outs:
        if dtype == "bf16":
            _close_bf16(got.cpu().view(torch.int16).numpy().view(np.uint16), ref, what)
        else:
            err = gpuio.rel_fro(got.cpu().numpy(), ref)
            assert err <= TOL, f"{what}: relative Frobenius error {err:.3e}"


def test_nvfp4_linear_is_reproducible_and_bf16_bypass():
    torch = gpuio.torch_cuda()
    from bit_microscaled_quantized_amd.module import NVFP4Linear
    x = torch.from_numpy(synth.normal(81, (256, 256))).cuda().to(torch.bfloat16)
    dy = torch.from_numpy(synth.normal(82, (256, 128)) * 1e-3).cuda().to(torch.bfloat16)
    grads = []
    for _ in range(2):
        layer = NVFP4Linear(256, 128, seed=5)
        xi = x.clone().requires_grad_(True)
        layer(xi).backward(dy)
        grads.append((xi.grad.clone(), layer.weight.grad.clone()))
    torch.cuda.synchronize()
    assert torch.equal(grads[0][0], grads[1][0]) and torch.equal(grads[0][1], grads[1][1])
    plain = NVFP4Linear(256, 128, seed=5, bf16=True)
    assert torch.equal(plain(x), torch.nn.functional.linear(x, plain.weight))


def test_nvfp4_linear_steady_state_adds_no_device_segment():
    """Once the first steps have filled PyTorch's cache, forward + backward
    take every buffer (quantized copies, GEMM outputs, split workspaces) from
    blocks it already holds: no new device segment, so no allocation call."""
    torch = gpuio.torch_cuda()
    from bit_microscaled_quantized_amd.module import NVFP4Linear
    x = torch.from_numpy(synth.normal(83, (512, 256))).cuda().to(torch.bfloat16)
    dy = torch.from_numpy(synth.normal(84, (512, 384)) * 1e-3).cuda().to(torch.bfloat16)
    layer = NVFP4Linear(256, 384, seed=7)

    def step():
        xi = x.clone().requires_grad_(True)
        layer(xi).backward(dy)
        layer.weight.grad = None

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["segment.all.allocated"]
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["segment.all.allocated"] == before


def test_nvfp4_linear_rejects_unsupported_shapes():
    torch = gpuio.torch_cuda()
    from bit_microscaled_quantized_amd.module import NVFP4Linear
    layer = NVFP4Linear(256, 128)
    with pytest.raises(ValueError, match="tokens"):
        layer(torch.zeros((100, 256), dtype=torch.bfloat16, device="cuda"))
