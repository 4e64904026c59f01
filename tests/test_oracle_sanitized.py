"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, CPU only): a C driver calls every oracle entry point on seeded inputs
of ragged shapes (full tensors and line ranges, every layout, RNE and SR,
bf16 and FP32, the RHT, MXFP4, dequantization, BF16 rounding, the FP64
contraction) and writes all outputs to one file.  The run must be free of
sanitizer reports, and its outputs must equal byte for byte those of the
ordinary build that the other tests load."""
import os
import subprocess

import numpy as np
import pytest

from bit_microscaled_quantized_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
int ora_quantize_range(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, int layout,
                       int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales, uint8_t *codes_t,
                       uint8_t *scales_t, float *ts, float *amax, int64_t b, int64_t e);
int ora_rht_quantize_range(const void *x, int dtype, int64_t tokens, int64_t cols, int64_t ld,
                           uint32_t mask, int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales,
                           float *ts, float *amax, int64_t b, int64_t e);
int ora_mx_quantize_range(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, int layout,
                          int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales, int64_t b, int64_t e);
void ora_mx_dequant(int64_t n, int64_t k, const uint8_t *codes, const uint8_t *scales, double *out);
void ora_dequant(int64_t n, int64_t k, const uint8_t *codes, const uint8_t *scales, int rowdiv,
                 float ts, double *out);
void ora_dequant_f32(int64_t n, int64_t k, const uint8_t *codes, const uint8_t *scales, int rowdiv,
                     float ts, float *out);
void ora_dequant_bf16(int64_t n, int64_t k, const uint8_t *codes, const uint8_t *scales, int rowdiv,
                      float ts, uint16_t *out);
void ora_bf16_rne_array(int64_t n, const float *x, uint16_t *out);
void ora_gemm_f64(int64_t M, int64_t N, int64_t K, const double *A, const double *B, double beta,
                  double *C);
void ora_block_scale_array(const float *amax_b, int64_t n, float s_enc, uint8_t *out);

static FILE *out;
static void put(const void *p, size_t n) { fwrite(p, 1, n, out); }

static void *slurp(const char *path, size_t n) {
  void *p = malloc(n);
  FILE *f = fopen(path, "rb");
  if (!f || fread(p, 1, n, f) != n) { fprintf(stderr, "cannot read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

int main(int argc, char **argv) {
  const int64_t R = atoll(argv[2]), C = atoll(argv[3]);
  char path[4096];
  snprintf(path, sizeof path, "%s/x16.bin", argv[1]);
  uint16_t *x16 = slurp(path, (size_t)(R * C * 2));
  snprintf(path, sizeof path, "%s/x32.bin", argv[1]);
  float *x32 = slurp(path, (size_t)(R * C * 4));
  snprintf(path, sizeof path, "%s/out.bin", argv[1]);
  out = fopen(path, "wb");
  const void *xs[2] = {x16, x32};
  for (int dt = 0; dt < 2; dt++)
    for (int layout = 0; layout < 3; layout++)
      for (int rnd = 0; rnd < 2; rnd++)
        for (int part = 0; part < 2; part++) {
          const int64_t n = R * C;
          uint8_t *codes = calloc(n / 2, 1), *scales = calloc(n / 16, 1);
          uint8_t *codes_t = layout == 2 ? calloc(n / 2, 1) : NULL;
          uint8_t *scales_t = layout == 2 ? calloc(n / 256, 1) : NULL;
          float ts = 0, am = 0;
          const int64_t lines = layout == 0 ? R : layout == 1 ? C : R / 16;
          const int64_t b = part ? lines / 3 : 0, e = part ? lines / 3 + 1 : INT64_MAX;
          if (ora_quantize_range(xs[dt], dt, R, C, C, layout, rnd, 1234567ull + rnd, codes, scales,
                                 codes_t, scales_t, &ts, &am, b, e)) return 3;
          put(codes, n / 2); put(scales, layout == 2 ? n / 256 : n / 16);
          if (codes_t) { put(codes_t, n / 2); put(scales_t, n / 256); }
          put(&ts, 4); put(&am, 4);
          if (!part) {
            const int64_t rr = layout == 1 ? C : R, cc = layout == 1 ? R : C;
            const int rowdiv = layout == 2 ? 16 : 1;
            double *d = malloc(n * 8);
            float *f = malloc(n * 4);
            uint16_t *h = malloc(n * 2);
            ora_dequant(rr, cc, codes, scales, rowdiv, ts, d);
            ora_dequant_f32(rr, cc, codes, scales, rowdiv, ts, f);
            ora_dequant_bf16(rr, cc, codes, scales, rowdiv, ts, h);
            put(d, n * 8); put(f, n * 4); put(h, n * 2);
            free(d); free(f); free(h);
          }
          free(codes); free(scales); free(codes_t); free(scales_t);
        }
  for (int dt = 0; dt < 2; dt++)
    for (int rnd = 0; rnd < 2; rnd++) {
      const int64_t n = R * C;
      uint8_t *codes = calloc(n / 2, 1), *scales = calloc(n / 16, 1);
      float ts = 0, am = 0;
      if (ora_rht_quantize_range(xs[dt], dt, R, C, C, 0xA5C3u, rnd, 99ull, codes, scales, &ts, &am, 0,
                                 INT64_MAX)) return 4;
      put(codes, n / 2); put(scales, n / 16); put(&ts, 4); put(&am, 4);
      free(codes); free(scales);
    }
  for (int layout = 0; layout < 2; layout++)
    for (int rnd = 0; rnd < 2; rnd++) {
      const int64_t n = R * C;
      uint8_t *codes = calloc(n / 2, 1), *scales = calloc(n / 32, 1);
      if (ora_mx_quantize_range(x32, 1, R, C, C, layout, rnd, 5ull, codes, scales, 0, INT64_MAX)) return 5;
      double *d = malloc(n * 8);
      ora_mx_dequant(layout ? C : R, layout ? R : C, codes, scales, d);
      put(codes, n / 2); put(scales, n / 32); put(d, n * 8);
      free(codes); free(scales); free(d);
    }
  {
    const int64_t n = R * C;
    uint16_t *h = malloc(n * 2);
    ora_bf16_rne_array(n, x32, h);
    put(h, n * 2);
    uint8_t *e = malloc(n);
    ora_block_scale_array(x32, n, 3.0f, e);
    put(e, n);
    free(h); free(e);
  }
  {
    const int64_t M = 16, N = 32, K = 48;
    double *A = malloc(M * K * 8), *B = malloc(N * K * 8), *Cm = malloc(M * N * 8);
    for (int64_t i = 0; i < M * K; i++) A[i] = x32[i];
    for (int64_t i = 0; i < N * K; i++) B[i] = x32[M * K + i];
    for (int64_t i = 0; i < M * N; i++) Cm[i] = 0.5;
    ora_gemm_f64(M, N, K, A, B, 1.0, Cm);
    put(Cm, M * N * 8);
    free(A); free(B); free(Cm);
  }
  fclose(out);
  free(x16); free(x32);
  return 0;
}
"""


def _expected(ora, x16, x32):
    R, C = x16.shape
    n = R * C
    parts = []
    for x in (x16, x32):
        for layout in (ora.ROW_1D, ora.COL_1D, ora.TILE_2D):
            for rnd in (ora.RNE, ora.SR):
                for part in (0, 1):
                    lines_n = R if layout == ora.ROW_1D else C if layout == ora.COL_1D else R // 16
                    rng = (lines_n // 3, lines_n // 3 + 1) if part else None
                    q = ora.quantize(x, layout, rnd, 1234567 + rnd, lines=rng)
                    parts += [q["codes"].tobytes(), q["scales"].tobytes()]
                    if layout == ora.TILE_2D:
                        parts += [q["codes_t"].tobytes(), q["scales_t"].tobytes()]
                    parts += [np.float32(q["tensor_scale"]).tobytes(), np.float32(q["amax"]).tobytes()]
                    if not part:
                        rowdiv = 16 if layout == ora.TILE_2D else 1
                        parts.append(ora.dequant(q["codes"], q["scales"], q["tensor_scale"], rowdiv).tobytes())
                        parts.append(ora.dequant_f32(q["codes"], q["scales"], q["tensor_scale"], rowdiv).tobytes())
                        parts.append(ora.dequant_bf16(q["codes"], q["scales"], q["tensor_scale"], rowdiv).tobytes())
    for x in (x16, x32):
        for rnd in (ora.RNE, ora.SR):
            q = ora.rht_quantize(x, 0xA5C3, rnd, 99)
            parts += [q["codes"].tobytes(), q["scales"].tobytes(), np.float32(q["tensor_scale"]).tobytes(),
                      np.float32(q["amax"]).tobytes()]
    for layout in (ora.ROW_1D, ora.COL_1D):
        for rnd in (ora.RNE, ora.SR):
            q = ora.mx_quantize(x32, layout, rnd, 5)
            parts += [q["codes"].tobytes(), q["scales"].tobytes(), ora.mx_dequant(q["codes"], q["scales"]).tobytes()]
    parts.append(ora.bf16_rne(x32).tobytes())
    parts.append(ora.block_scale_array(x32, 3.0).tobytes())
    A = x32.reshape(-1)[:16 * 48].astype(np.float64).reshape(16, 48)
    B = x32.reshape(-1)[16 * 48:16 * 48 + 32 * 48].astype(np.float64).reshape(32, 48)
    parts.append(ora.gemm_f64_loop(A, B, np.full((16, 32), 0.5), 1.0).tobytes())
    return b"".join(parts)


@pytest.mark.parametrize("shape", [(64, 96), (160, 224)])
def test_oracle_under_asan_ubsan(ora, tmp_path, shape):
    probe = subprocess.run(["gcc", "-fsanitize=address,undefined", "-x", "c", "-", "-o", os.devnull],
                           input="int main(void){return 0;}", capture_output=True, text=True)
    if probe.returncode != 0:
        pytest.skip("gcc has no ASan/UBSan here")
    R, C = shape
    x32 = synth.lognormal_signed(11 + R, (R, C))
    x32[3, 5] = 0.0
    x32[4, :16] = 0.0  # an empty block
    x32[7, 7] = -0.0
    x16 = synth.f32_to_bf16_bits(synth.student_t(12 + R, (R, C)))
    x16.tofile(tmp_path / "x16.bin")
    x32.tofile(tmp_path / "x32.bin")
    drv = tmp_path / "drv.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "drv"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe), str(drv),
           ORACLE_C, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), str(tmp_path), str(R), str(C)], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    got = (tmp_path / "out.bin").read_bytes()
    want = _expected(ora, x16, x32)
    assert len(got) == len(want)
    assert got == want
