"""The fp64 oracle built with gcc under AddressSanitizer and
UndefinedBehaviorSanitizer, driven by a small C program over every entry
point, storage type and edge length (empty, negative and over-long seqlens,
full caches, windows wider and narrower than the sequence, listed prefill
rows). Every buffer is its own heap allocation of exactly the documented
size, so a read or write past any of them, a double free or a leak fails the
run; the C program also checks a few exact properties on the way (rows sum to
one, one cached position returns its value row, the append writes exactly
one cache row)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "gqa_oracle.c")

DRIVER = r'''
#include <assert.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_group_of_head(int h0, int H, int G);
double oracle_kv_cache_bytes_per_token(int kv_heads, int d_h, int layers, int bytes_per_scalar);
void oracle_decode(const void *q, const void *k, const void *v, int dtype, const int32_t *seqlens,
                   int B, int H, int G, int D, int Tmax, double scale, double *out, double *probs);
void oracle_prefill(const void *q, const void *k, const void *v, int dtype, int B, int T, int H,
                    int G, int D, int causal, const int32_t *rows_b, const int32_t *rows_t,
                    const int32_t *rows_h, int64_t n_rows, double *out);
void oracle_decode_step(const void *q, const void *k_new, const void *v_new, void *k, void *v, int dtype,
                        const int32_t *seqlens, int B, int H, int G, int D, int Tmax, double scale, int window,
                        double *out);
void oracle_prefill_window(const void *q, const void *k, const void *v, int dtype, int B, int T, int H,
                           int G, int D, int window, const int32_t *rows_b, const int32_t *rows_t,
                           const int32_t *rows_h, int64_t n_rows, double *out);
void oracle_weighted_pool(const void *in, int dtype, int64_t N, int H, int G, int D, const double *w,
                          double *out);
void oracle_mean_pool(const void *in, int dtype, int64_t N, int H, int G, int D, double *out);
void oracle_set_threads(int n);

static uint64_t rng = 88172645463325252ull;
static double unif(void) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (rng >> 11) * 0x1p-53; }
static size_t esize(int dt) { return dt == 0 || dt == 3 ? 2 : dt == 1 ? 4 : 8; }

/* n elements of storage type dt with values in [-2, 2) (finite, no NaN) */
static void *fill(size_t n, int dt) {
  void *p = malloc(n * esize(dt) + (n == 0));
  for (size_t i = 0; i < n; ++i) {
    double x = 4.0 * unif() - 2.0;
    if (dt == 2) ((double *)p)[i] = x;
    else if (dt == 1) ((float *)p)[i] = (float)x;
    else if (dt == 0) { float f = (float)x; uint32_t u; memcpy(&u, &f, 4); ((uint16_t *)p)[i] = (uint16_t)(u >> 16); }
    else { /* fp16: sign, 5-bit exponent 13..16 (|x| in [0.25, 4)), random fraction */
      uint16_t s = unif() < 0.5 ? 0x8000 : 0, e = (uint16_t)(13 + (int)(unif() * 3)), f = (uint16_t)(unif() * 1024);
      ((uint16_t *)p)[i] = (uint16_t)(s | (e << 10) | f); }
  }
  return p;
}
static void finite(const double *x, size_t n) { for (size_t i = 0; i < n; ++i) assert(isfinite(x[i])); }

int main(void) {
  oracle_set_threads(4);
  assert(oracle_kv_cache_bytes_per_token(64, 128, 80, 2) == 2621440.0);
  const int shapes[][4] = {{1, 1, 1, 64}, {2, 8, 2, 64}, {3, 12, 3, 128}, {2, 6, 6, 64}, {1, 16, 1, 128}};
  for (int si = 0; si < 5; ++si) for (int dt = 0; dt < 4; ++dt) {
    const int B = shapes[si][0], H = shapes[si][1], G = shapes[si][2], D = shapes[si][3];
    for (int h = 0; h < H; ++h) { int g = oracle_group_of_head(h, H, G); assert(g >= 0 && g < G); }
    for (int Tmax = 0; Tmax <= 9; Tmax += 3) {
      const size_t nq = (size_t)B * H * D, nkv = (size_t)B * Tmax * G * D, nn = (size_t)B * G * D;
      int32_t *sl = malloc(sizeof(int32_t) * B);
      const int32_t pick[] = {-3, 0, 1, Tmax - 1, Tmax, Tmax + 5};
      for (int b = 0; b < B; ++b) sl[b] = pick[(b + si + Tmax) % 6];
      void *q = fill(nq, dt), *k = fill(nkv, dt), *v = fill(nkv, dt), *kn = fill(nn, dt), *vn = fill(nn, dt);
      double *out = malloc(sizeof(double) * (nq + 1)), *probs = malloc(sizeof(double) * ((size_t)B * H * Tmax + 1));
      oracle_decode(q, k, v, dt, sl, B, H, G, D, Tmax, 0.125, out, probs);
      finite(out, nq);
      for (int r = 0; r < B * H; ++r) {
        int L = sl[r / H] < 0 ? 0 : sl[r / H] > Tmax ? Tmax : sl[r / H];
        double s = 0; for (int t = 0; t < Tmax; ++t) s += probs[(size_t)r * Tmax + t];
        if (L > 0) assert(fabs(s - 1.0) < 1e-12); else assert(s == 0.0);
      }
      for (int w = 0; w <= 4; w += 2) {
        void *k2 = malloc(nkv * esize(dt) + 1), *v2 = malloc(nkv * esize(dt) + 1);
        memcpy(k2, k, nkv * esize(dt)); memcpy(v2, v, nkv * esize(dt));
        oracle_decode_step(q, kn, vn, k2, v2, dt, sl, B, H, G, D, Tmax, 0.125, w, out);
        finite(out, nq);
        size_t changed = 0;
        for (size_t i = 0; i < nkv * esize(dt); ++i) changed += ((char *)k2)[i] != ((char *)k)[i];
        size_t appended = 0;
        for (int b = 0; b < B; ++b) { int L = sl[b] < 0 ? 0 : sl[b] > Tmax ? Tmax : sl[b]; appended += L < Tmax; }
        assert(changed <= appended * G * D * esize(dt));
        oracle_decode_step(q, NULL, NULL, k2, v2, dt, sl, B, H, G, D, Tmax, 0.125, w, out);
        finite(out, nq);
        free(k2); free(v2);
      }
      free(sl); free(q); free(k); free(v); free(kn); free(vn); free(out); free(probs);
    }
    /* one cached position returns its value row exactly (fp64 storage) */
    if (dt == 2) {
      const size_t nq = (size_t)B * H * D, nkv = (size_t)B * 1 * G * D;
      int32_t *sl = malloc(sizeof(int32_t) * B);
      for (int b = 0; b < B; ++b) sl[b] = 1;
      double *q = fill(nq, 2), *k = fill(nkv, 2), *v = fill(nkv, 2), *out = malloc(sizeof(double) * nq);
      oracle_decode(q, k, v, 2, sl, B, H, G, D, 1, 0.3, out, NULL);
      for (int b = 0; b < B; ++b) for (int h = 0; h < H; ++h) for (int d = 0; d < D; ++d)
        assert(out[((size_t)b * H + h) * D + d] == v[((size_t)b * G + oracle_group_of_head(h, H, G)) * D + d]);
      free(sl); free(q); free(k); free(v); free(out);
    }
    for (int T = 1; T <= 7; T += 3) {
      const size_t nq = (size_t)B * T * H * D, nkv = (size_t)B * T * G * D;
      void *q = fill(nq, dt), *k = fill(nkv, dt), *v = fill(nkv, dt);
      double *out = malloc(sizeof(double) * nq);
      for (int causal = 0; causal < 2; ++causal) { oracle_prefill(q, k, v, dt, B, T, H, G, D, causal, NULL, NULL, NULL, 0, out); finite(out, nq); }
      for (int w = 0; w <= 3; ++w) { oracle_prefill_window(q, k, v, dt, B, T, H, G, D, w, NULL, NULL, NULL, 0, out); finite(out, nq); }
      int32_t rb[3] = {B - 1, 0, B - 1}, rt[3] = {T - 1, 0, T / 2}, rh[3] = {H - 1, 0, H / 2};
      double *rows = malloc(sizeof(double) * 3 * D);
      oracle_prefill(q, k, v, dt, B, T, H, G, D, 1, rb, rt, rh, 3, rows); finite(rows, 3 * (size_t)D);
      oracle_prefill_window(q, k, v, dt, B, T, H, G, D, 2, rb, rt, rh, 3, rows); finite(rows, 3 * (size_t)D);
      free(q); free(k); free(v); free(out); free(rows);
    }
    for (int N = 0; N <= 5; N += 5) {
      void *in = fill((size_t)N * H * D, dt);
      double *w = malloc(sizeof(double) * H), *out = malloc(sizeof(double) * ((size_t)N * G * D + 1));
      for (int h = 0; h < H; ++h) w[h] = unif();
      oracle_mean_pool(in, dt, N, H, G, D, out); finite(out, (size_t)N * G * D);
      oracle_weighted_pool(in, dt, N, H, G, D, w, out); finite(out, (size_t)N * G * D);
      free(in); free(w); free(out);
    }
  }
  puts("ok");
  return 0;
}
'''


def test_oracle_under_asan_ubsan(tmp_path):
    src = tmp_path / "drive.c"
    src.write_text(DRIVER)
    exe = tmp_path / "drive"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    str(src), ORACLE_C, "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="4")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]
