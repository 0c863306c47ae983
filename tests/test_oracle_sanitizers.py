"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
only): a small C driver links ar_oracle.c built with -fsanitize=address,undefined
and exercises every entry point, including empty inputs, one-element rows,
in-place aliasing and rejected arguments. Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r'''
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
int oracle_ar_sum(int, int, const void *const *, size_t, void *);
int oracle_rmsnorm(int, size_t, int, const void *, const void *, float, void *);
int oracle_ar_residual_rmsnorm(int, int, const void *const *, size_t, int, const void *, const void *,
                               const void *, float, void *, void *);
static unsigned long long st = 88172645463325252ull;
static unsigned next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (unsigned)st; }
int main(void) {
  for (int dt = 0; dt < 3; ++dt) {
    size_t s = dt == 0 ? 4 : 2;
    for (int R = 1; R <= 8; ++R) {
      size_t sizes[] = {0, 1, 7, 64, 1000};
      for (int k = 0; k < 5; ++k) {
        size_t n = sizes[k];
        void *p[8]; for (int r = 0; r < R; ++r) { p[r] = malloc(n * s + 1); for (size_t i = 0; i < n * s; ++i) ((unsigned char *)p[r])[i] = (unsigned char)next(); }
        void *out = malloc(n * s + 1);
        if (oracle_ar_sum(dt, R, (const void *const *)p, n, out)) return 1;
        if (oracle_ar_sum(dt, R, (const void *const *)p, n, p[0])) return 2;  /* in place */
        int H = n ? (int)(n % 8 == 0 ? 8 : 1) : 1;
        void *w = malloc(H * s), *b = malloc(H * s), *q = malloc(n * s + 1), *inter = malloc(n * s + 1);
        for (size_t i = 0; i < H * s; ++i) { ((unsigned char *)w)[i] = (unsigned char)next(); ((unsigned char *)b)[i] = (unsigned char)next(); }
        for (size_t i = 0; i < n * s; ++i) ((unsigned char *)q)[i] = (unsigned char)next();
        if (oracle_ar_residual_rmsnorm(dt, R, (const void *const *)p, n, H, b, q, w, 1e-6f, out, inter)) return 3;
        if (oracle_ar_residual_rmsnorm(dt, R, (const void *const *)p, n, H, NULL, NULL, w, 0.0f, out, inter)) return 4;
        if (oracle_ar_residual_rmsnorm(dt, R, (const void *const *)p, n, H, b, q, w, 1e-5f, out, q)) return 5;  /* intermediate == residual */
        if (oracle_rmsnorm(dt, n, H, out, w, 1e-5f, out)) return 6;  /* in place */
        if (n && oracle_ar_residual_rmsnorm(dt, R, (const void *const *)p, n, (int)n + 1, b, q, w, 0.f, out, inter) == 0) return 7;
        if (oracle_ar_sum(dt, 0, (const void *const *)p, n, out) == 0) return 8;
        free(w); free(b); free(q); free(inter); free(out);
        for (int r = 0; r < R; ++r) free(p[r]);
      }
    }
  }
  if (oracle_ar_sum(5, 2, NULL, 4, NULL) == 0) return 9;
  return 0;
}
'''


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", str(exe), str(drv),
           os.path.join(ROOT, "oracle", "ar_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
