"""Host-side checks of libnvfp4 that need no GPU: the library loads, exports
exactly the entry points include/nvfp4.h declares, and rejects bad arguments
with the documented status codes before anything is enqueued."""
import os
import re
import subprocess

import pytest

import bit_microscaled_quantized_amd as nv
from bit_microscaled_quantized_amd import nvfp4 as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


def declared_symbols():
    text = "".join(open(os.path.join(os.path.dirname(HEADER), f)).read()
                   for f in sorted(os.listdir(os.path.dirname(HEADER))) if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:nvfp4_status|const char \*)\s*((?:nvfp4|mxfp4)_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(b.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = nv.load_library()
    for s in declared_symbols():
        assert hasattr(lib, s), s
    out = subprocess.run(["nm", "-D", "--defined-only", nv.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported_c = sorted({line.split()[-1] for line in out.splitlines()
                         if line.split()[-1].startswith(("nvfp4_", "mxfp4_"))})
    assert exported_c == declared_symbols()


def _declarations():
    """name -> (return type, [parameter types]) of every entry point in include/*.h."""
    text = "".join(open(os.path.join(os.path.dirname(HEADER), f)).read()
                   for f in sorted(os.listdir(os.path.dirname(HEADER))) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    out = {}
    for ret, name, params in re.findall(r"^\s*(nvfp4_status|const char \*)\s*((?:nvfp4|mxfp4)_\w+)\s*\(([^)]*)\)\s*;",
                                        text, re.M):
        types = []
        for p in params.split(","):
            p = " ".join(p.split())
            m = re.match(r"^(.*?)(\w+)$", p)
            assert m, (name, p)
            types.append(m.group(1).replace(" ", ""))
        out[name] = (ret.replace(" ", ""), types)
    return out


def test_binding_argument_types_match_the_header():
    """Each entry point's ctypes argument and return types are the C types
    the header declares, in order (so no argument is marshalled at another
    width or position)."""
    import ctypes
    lib = nv.load_library()
    scalar = {"int64_t": ctypes.c_int64, "uint64_t": ctypes.c_uint64, "uint32_t": ctypes.c_uint32,
              "int32_t": ctypes.c_int32, "int": ctypes.c_int32, "float": ctypes.c_float}
    decls = _declarations()
    assert sorted(decls) == sorted(b.EXPORTED)
    for name, (ret, types) in decls.items():
        fn = getattr(lib, name)
        want = []
        for t in types:
            if t == "int64_t*":
                want.append(ctypes.POINTER(ctypes.c_int64))
            elif t.endswith("*"):
                want.append(ctypes.c_void_p)
            else:
                want.append(scalar[t.replace("const", "")])
        assert list(fn.argtypes) == want, (name, types, fn.argtypes)
        assert fn.restype == (ctypes.c_char_p if ret == "constchar*" else ctypes.c_int32), name


def test_mxfp4_argument_errors():
    def q(**kw):
        args = dict(x=FAKE, dt=0, rows=32, cols=64, ld_x=64, layout=0, rnd=0, seed=0, codes=FAKE,
                    scales=FAKE)
        args.update(kw)
        return nv.mxfp4_quantize(**args, stream=0, raise_on_error=False)
    assert q(codes=None) == b.NVFP4_EINVAL
    assert q(layout=2) == b.NVFP4_EINVAL                 # no 2D layout for MXFP4
    assert q(rnd=3) == b.NVFP4_EINVAL
    assert q(cols=48, ld_x=48) == b.NVFP4_ESHAPE         # row blocks need cols % 32
    assert q(layout=1, rows=48) == b.NVFP4_ESHAPE        # column blocks need rows % 32
    assert q(codes=FAKE + 4) == b.NVFP4_EALIGN
    assert q(scales=FAKE + 2) == b.NVFP4_EALIGN

    def g(**kw):
        args = dict(M=256, N=256, K=256, a_codes=FAKE, a_scales=FAKE, b_codes=FAKE, b_scales=FAKE,
                    c=FAKE, ldc=256, beta=0.0)
        args.update(kw)
        return nv.mxfp4_gemm(**args, stream=0, raise_on_error=False)
    assert g(b_scales=None) == b.NVFP4_EINVAL
    assert g(beta=2.0) == b.NVFP4_EINVAL
    assert g(K=64) == b.NVFP4_ESHAPE                     # K must be a multiple of 128
    assert g(M=8) == b.NVFP4_ESHAPE
    assert g(ldc=100) == b.NVFP4_ESHAPE
    assert g(a_scales=FAKE + 1) == b.NVFP4_EALIGN
    assert g(c=FAKE + 8) == b.NVFP4_EALIGN


def test_status_strings():
    assert nv.nvfp4_status_str(0) == "NVFP4_OK"
    for s in range(1, 5):
        assert nv.nvfp4_status_str(s).startswith("NVFP4_E")
    assert "unknown" in nv.nvfp4_status_str(99)


def q(**kw):
    args = dict(x=FAKE, dt=0, rows=32, cols=32, ld_x=32, layout=0, rnd=0, seed=0, codes=FAKE,
                scales=FAKE, codes_t=None, scales_t=None, tensor_scale=FAKE, amax=FAKE)
    args.update(kw)
    return nv.nvfp4_quantize(**args, stream=0, raise_on_error=False)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), b.NVFP4_EINVAL),
    (dict(codes=None), b.NVFP4_EINVAL),
    (dict(amax=None), b.NVFP4_EINVAL),
    (dict(dt=7), b.NVFP4_EINVAL),
    (dict(layout=3), b.NVFP4_EINVAL),
    (dict(rnd=2), b.NVFP4_EINVAL),
    (dict(codes_t=FAKE, scales_t=FAKE), b.NVFP4_EINVAL),          # transposed outputs on a 1D layout
    (dict(layout=2, codes_t=FAKE), b.NVFP4_EINVAL),               # codes_t without scales_t
    (dict(rows=24), b.NVFP4_ESHAPE),
    (dict(cols=8, ld_x=8), b.NVFP4_ESHAPE),
    (dict(rows=0), b.NVFP4_ESHAPE),
    (dict(ld_x=16), b.NVFP4_ESHAPE),
    (dict(rows=1 << 20, cols=1 << 12, ld_x=1 << 12), b.NVFP4_ESHAPE),  # 2^32 elements
    (dict(x=FAKE + 4), b.NVFP4_EALIGN),
    (dict(ld_x=36), b.NVFP4_EALIGN),                              # 72-byte bf16 rows
    (dict(codes=FAKE + 8), b.NVFP4_EALIGN),
    (dict(tensor_scale=FAKE + 2), b.NVFP4_EALIGN),
])
def test_quantize_argument_errors(kw, status):
    assert q(**kw) == status


def test_rht_quantize_argument_errors():
    def r(**kw):
        args = dict(x=FAKE, dt=0, tokens=32, cols=32, ld_x=32, sign_mask=0, rnd=0, seed=0,
                    codes=FAKE, scales=FAKE, tensor_scale=FAKE, amax=FAKE)
        args.update(kw)
        return nv.nvfp4_rht_quantize(**args, stream=0, raise_on_error=False)
    assert r(x=None) == b.NVFP4_EINVAL
    assert r(rnd=5) == b.NVFP4_EINVAL
    assert r(tokens=40) == b.NVFP4_ESHAPE
    assert r(cols=20, ld_x=20) == b.NVFP4_ESHAPE
    assert r(scales=FAKE + 1) == b.NVFP4_EALIGN


def test_quantize_row_rht_argument_errors():
    def r(**kw):
        args = dict(x=FAKE, dt=0, tokens=32, cols=32, ld_x=32, row_rnd=0, row_seed=0, row_codes=FAKE,
                    row_scales=FAKE, row_tensor_scale=FAKE, row_amax=FAKE, sign_mask=0, rht_rnd=1,
                    rht_seed=0, rht_codes=FAKE, rht_scales=FAKE, rht_tensor_scale=FAKE, rht_amax=FAKE)
        args.update(kw)
        return nv.nvfp4_quantize_row_rht(**args, stream=0, raise_on_error=False)
    assert r(x=None) == b.NVFP4_EINVAL
    assert r(rht_codes=None) == b.NVFP4_EINVAL
    assert r(row_amax=None) == b.NVFP4_EINVAL
    assert r(row_rnd=2) == b.NVFP4_EINVAL
    assert r(rht_rnd=-1) == b.NVFP4_EINVAL
    assert r(tokens=40) == b.NVFP4_ESHAPE
    assert r(cols=20, ld_x=20) == b.NVFP4_ESHAPE
    assert r(rht_scales=FAKE + 1) == b.NVFP4_EALIGN
    assert r(row_tensor_scale=FAKE + 2) == b.NVFP4_EALIGN


def g(**kw):
    args = dict(M=256, N=256, K=256, a_codes=FAKE, a_scales=FAKE, a_tensor_scale=FAKE, b_codes=FAKE,
                b_scales=FAKE, b_scale_rowdiv=1, b_tensor_scale=FAKE, c=FAKE, ldc=256, beta=0.0)
    args.update(kw)
    return nv.nvfp4_gemm(**args, stream=0, raise_on_error=False)


@pytest.mark.parametrize("kw,status", [
    (dict(a_codes=None), b.NVFP4_EINVAL),
    (dict(c=None), b.NVFP4_EINVAL),
    (dict(b_scale_rowdiv=4), b.NVFP4_EINVAL),
    (dict(beta=0.5), b.NVFP4_EINVAL),
    (dict(M=250), b.NVFP4_ESHAPE),
    (dict(N=8), b.NVFP4_ESHAPE),
    (dict(K=96), b.NVFP4_ESHAPE),
    (dict(K=0), b.NVFP4_ESHAPE),
    (dict(ldc=128), b.NVFP4_ESHAPE),
    (dict(M=1 << 20, K=1 << 13), b.NVFP4_ESHAPE),                  # A codes of 4 GiB
    (dict(N=1 << 20, K=1 << 13, ldc=1 << 20), b.NVFP4_ESHAPE),     # B codes of 4 GiB
    (dict(a_codes=FAKE + 4), b.NVFP4_EALIGN),
    (dict(c=FAKE + 4), b.NVFP4_EALIGN),
    (dict(ldc=258), b.NVFP4_EALIGN),
    (dict(workspace=FAKE + 4, workspace_bytes=1 << 20), b.NVFP4_EALIGN),
    (dict(workspace=FAKE, workspace_bytes=-1), b.NVFP4_ESHAPE),
])
def test_gemm_argument_errors(kw, status):
    assert g(**kw) == status


@pytest.mark.parametrize("M,N,K", [(250, 256, 256), (256, 8, 256), (256, 256, 96), (0, 256, 256)])
def test_gemm_workspace_size_shape_errors(M, N, K):
    import ctypes
    out = ctypes.c_int64(-7)
    assert b.load_library().nvfp4_gemm_workspace_size(M, N, K, ctypes.byref(out)) == b.NVFP4_ESHAPE
    assert out.value == -7  # untouched on error
    assert b.load_library().nvfp4_gemm_workspace_size(256, 256, 256, None) == b.NVFP4_EINVAL


def test_errors_raise_in_checked_mode():
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm(256, 256, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 256, 0.0, stream=0)
    assert e.value.status == b.NVFP4_ESHAPE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "_LIB_PATH", str(tmp_path / "libnvfp4.so"))
    with pytest.raises(RuntimeError, match="missing"):
        b.load_library()


def test_dequantize_argument_errors():
    def d(**kw):
        args = dict(codes=FAKE, scales=FAKE, scale_rowdiv=1, tensor_scale=FAKE, rows=32, cols=64,
                    out_dt=b.NVFP4_BF16, out=FAKE, ld_out=64)
        args.update(kw)
        return nv.nvfp4_dequantize(**args, stream=0, raise_on_error=False)
    assert d(codes=None) == b.NVFP4_EINVAL
    assert d(out=None) == b.NVFP4_EINVAL
    assert d(scale_rowdiv=4) == b.NVFP4_EINVAL
    assert d(out_dt=7) == b.NVFP4_EINVAL
    assert d(cols=40, ld_out=40) == b.NVFP4_ESHAPE        # cols % 16
    assert d(rows=24, scale_rowdiv=16) == b.NVFP4_ESHAPE  # 2D tile grid needs rows % 16
    assert d(ld_out=32) == b.NVFP4_ESHAPE
    assert d(rows=0) == b.NVFP4_ESHAPE
    assert d(codes=FAKE + 8) == b.NVFP4_EALIGN
    assert d(out=FAKE + 4) == b.NVFP4_EALIGN
    assert d(ld_out=68) == b.NVFP4_EALIGN                 # 136-byte BF16 rows


def test_gemm_bf16_argument_errors():
    def g16(**kw):
        args = dict(M=256, N=256, K=256, a_codes=FAKE, a_scales=FAKE, a_tensor_scale=FAKE,
                    b_codes=FAKE, b_scales=FAKE, b_scale_rowdiv=1, b_tensor_scale=FAKE, c=FAKE,
                    ldc=256, beta=0.0)
        args.update(kw)
        return nv.nvfp4_gemm_bf16(**args, stream=0, raise_on_error=False)
    assert g16(c=None) == b.NVFP4_EINVAL
    assert g16(beta=0.5) == b.NVFP4_EINVAL
    assert g16(K=96) == b.NVFP4_ESHAPE
    assert g16(ldc=260) == b.NVFP4_EALIGN                 # BF16 rows must be 16-byte multiples
    assert g16(c=FAKE + 8) == b.NVFP4_EALIGN


def test_gemm_noalloc_argument_errors():
    def gn(**kw):
        args = dict(M=256, N=256, K=256, a_codes=FAKE, a_scales=FAKE, a_tensor_scale=FAKE,
                    b_codes=FAKE, b_scales=FAKE, b_scale_rowdiv=1, b_tensor_scale=FAKE, c=FAKE,
                    ldc=256, beta=0.0)
        args.update(kw)
        return nv.nvfp4_gemm_noalloc(**args, stream=0, raise_on_error=False)
    assert gn(a_codes=None) == b.NVFP4_EINVAL
    assert gn(b_tensor_scale=None) == b.NVFP4_EINVAL
    assert gn(b_scale_rowdiv=8) == b.NVFP4_EINVAL
    assert gn(beta=2.0) == b.NVFP4_EINVAL
    assert gn(K=96) == b.NVFP4_ESHAPE
    assert gn(ldc=128) == b.NVFP4_ESHAPE
    assert gn(M=1 << 20, K=1 << 13) == b.NVFP4_ESHAPE
    assert gn(c=FAKE + 4) == b.NVFP4_EALIGN
    assert gn(ldc=258) == b.NVFP4_EALIGN
    assert "static" in nv.nvfp4_status_str(b.NVFP4_ESCRATCH)


def test_single_pass_controls():
    L = b.load_library()
    assert L.nvfp4_set_quantize_passes(1) == b.NVFP4_EINVAL
    assert L.nvfp4_set_quantize_passes(3) == b.NVFP4_EINVAL
    assert L.nvfp4_set_quantize_passes(2) == b.NVFP4_OK
    assert L.nvfp4_set_quantize_passes(0) == b.NVFP4_OK
    assert L.nvfp4_set_sync_spin_limit(-1) == b.NVFP4_EINVAL
    assert L.nvfp4_set_sync_spin_limit(1 << 24) == b.NVFP4_OK
    assert L.nvfp4_single_pass_stats(None, None) == b.NVFP4_EINVAL
