"""The C oracles built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) and run on small cases by a driver program: no
out-of-bounds access, leak or undefined behaviour in the checker itself.  CPU
only."""
import os
import shutil
import subprocess

import pytest

from oracle import build as oracle_build

DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
int xattn_ref_run(const double*, const double*, const double*, const double*, double*, double*,
                  double*, double*, double*, int, int, int, int, int, double, int, int);
int xattn_ref_decode(const double*, const double*, const double*, const int*, double*, double*,
                     int, int, int, int, int, double);
int xattn_ref_qknorm_rope_fwd(const double*, const double*, double*, int, int, int, int, double,
                              double);
int xattn_ref_qknorm_rope_bwd(const double*, const double*, const double*, double*, double*, int,
                              int, int, int, double, double);
static double* arr(size_t n, unsigned seed) {
  double* a = (double*)malloc(n * sizeof(double));
  srand(seed);
  for (size_t i = 0; i < n; ++i) a[i] = (double)rand() / RAND_MAX - 0.5;
  return a;
}
int main(void) {
  const int B = 2, S = 9, H = 4, Hkv = 2, hd = 8;
  const size_t nq = (size_t)B * H * S * hd, nk = (size_t)B * Hkv * S * hd;
  double *q = arr(nq, 1), *k = arr(nk, 2), *v = arr(nk, 3), *dO = arr(nq, 4);
  double *o = arr(nq, 5), *lse = arr((size_t)B * H * S, 6), *dq = arr(nq, 7);
  double *dk = arr(nk, 8), *dv = arr(nk, 9);
  int rc = xattn_ref_run(q, k, v, dO, o, lse, dq, dk, dv, B, S, H, Hkv, hd, 0.3, 0, B * Hkv);
  const int lens[2] = {9, 0};
  double *qd = arr((size_t)B * H * hd, 10), *od = arr((size_t)B * H * hd, 11), *ld = arr(B * H, 12);
  rc |= xattn_ref_decode(qd, k, v, lens, od, ld, B, S, H, Hkv, hd, 0.3);
  double *x = arr(nq, 13), *w = arr(hd, 14), *out = arr(nq, 15), *g = arr(nq, 16);
  double *dx = arr(nq, 17), *dw = arr(hd, 18);
  rc |= xattn_ref_qknorm_rope_fwd(x, w, out, B, S, H, hd, 1e-6, 10000.0);
  rc |= xattn_ref_qknorm_rope_bwd(x, w, g, dx, dw, B, S, H, hd, 1e-6, 10000.0);
  double s = 0;
  for (size_t i = 0; i < nq; ++i) s += o[i] + dq[i] + out[i] + dx[i];
  free(q); free(k); free(v); free(dO); free(o); free(lse); free(dq); free(dk); free(dv);
  free(qd); free(od); free(ld); free(x); free(w); free(out); free(g); free(dx); free(dw);
  printf("rc=%d sum=%g\n", rc, s);
  return rc != 0 || !isfinite(s);
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracles_clean_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    srcs = [oracle_build.SRC, oracle_build.SRC_DEC, oracle_build.SRC_NORM]
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
           str(drv), *srcs, "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "rc=0" in r.stdout
