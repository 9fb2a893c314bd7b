"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (host only).

A small C driver calls orc_indexer_scores, orc_topk, orc_block_topk and orc_attention on edge cases (a single
visible key, k larger than the visible count, -1 padding in the index rows, a shared latent row
as well as a separate V, grouped kv heads) and checks a few facts the definitions fix; the whole
program is built with gcc -fsanitize=address,undefined, so any out-of-bounds access, leak or
undefined arithmetic fails the test.
"""
import os
import shutil
import subprocess

import pytest

ORACLE_C = os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", "oracle", "oracle.c")

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_indexer_scores(const float *q, const float *w, const float *k, const int64_t *visible,
                        int64_t n_q, int64_t n_k, int H_I, int d_I, double *out, double *abs_out);
void orc_topk(const double *scores, int64_t ld, const int64_t *visible, const int32_t *k_per_row,
              int64_t n_q, int32_t k_max, int32_t *idx);
void orc_block_topk(const double *scores, int64_t ld, const int64_t *visible, const int32_t *k_per_row,
                    int64_t n_q, int32_t k_max, int64_t block_size, int64_t n_blocks, int32_t *idx,
                    int32_t *blocks_out);
void orc_attention(const float *q, const float *K, const float *V, const int32_t *idx, int64_t idx_ld,
                   int64_t n_q, int64_t n_k, int H, int H_kv, int d_qk, int d_v, double scale,
                   double *out, double *lse);

static uint32_t state = 12345u;
static float draw(void) { state = state * 1664525u + 1013904223u; return ((int)(state >> 8) - (1 << 23)) / (float)(1 << 23); }
static float *randv(size_t n) { float *p = malloc(n * sizeof(float)); for (size_t i = 0; i < n; ++i) p[i] = draw(); return p; }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); return 1; } } while (0)

static int run_case(int64_t n_q, int64_t n_k, int H_I, int d_I, int k_max, int H, int H_kv, int d_qk, int d_v, int sep_v)
{
    float *q_i = randv((size_t)(n_q * H_I * d_I)), *w = randv((size_t)(n_q * H_I)), *k_i = randv((size_t)(n_k * d_I));
    int64_t *vis = malloc((size_t)n_q * sizeof(int64_t));
    int32_t *kr = malloc((size_t)n_q * sizeof(int32_t));
    for (int64_t i = 0; i < n_q; ++i) { vis[i] = 1 + (i * 7) % n_k; kr[i] = 1 + (int32_t)((i * 5) % k_max); }
    double *s = malloc((size_t)(n_q * n_k) * sizeof(double)), *a = malloc((size_t)(n_q * n_k) * sizeof(double));
    orc_indexer_scores(q_i, w, k_i, vis, n_q, n_k, H_I, d_I, s, a);
    for (int64_t i = 0; i < n_q; ++i)
        for (int64_t j = 0; j < n_k; ++j) {
            if (j < vis[i]) { CHECK(isfinite(s[i * n_k + j])); CHECK(fabs(s[i * n_k + j]) <= a[i * n_k + j] + 1e-12); }
            else CHECK(isinf(s[i * n_k + j]) && s[i * n_k + j] < 0);
        }
    int32_t *idx = malloc((size_t)(n_q * k_max) * sizeof(int32_t));
    for (int per_row = 0; per_row < 2; ++per_row) {
        orc_topk(s, n_k, vis, per_row ? kr : NULL, n_q, k_max, idx);
        for (int64_t i = 0; i < n_q; ++i) {
            int64_t m = per_row ? kr[i] : k_max;
            if (m > vis[i]) m = vis[i];
            for (int r = 0; r < k_max; ++r) {
                int32_t v = idx[i * k_max + r];
                if (r < m) CHECK(v >= 0 && v < vis[i]); else CHECK(v == -1);
            }
        }
    }
    /* two-tier selection: blocks of 3 tokens (a short last block on most rows), more blocks
       asked for than some rows have */
    int32_t *blk = malloc((size_t)(n_q * 4) * sizeof(int32_t));
    for (int per_row = 0; per_row < 2; ++per_row) {
        orc_block_topk(s, n_k, vis, per_row ? kr : NULL, n_q, k_max, 3, 4, idx, blk);
        for (int64_t i = 0; i < n_q; ++i) {
            int64_t n_blk = (vis[i] + 2) / 3, kept = n_blk < 4 ? n_blk : 4;
            for (int r = 0; r < 4; ++r) {
                int32_t b = blk[i * 4 + r];
                if (r < kept) CHECK(b >= 0 && b < n_blk); else CHECK(b == -1);
            }
            int nsel = 0;
            for (int r = 0; r < k_max; ++r) {
                int32_t v = idx[i * k_max + r];
                if (v < 0) { CHECK(v == -1); continue; }
                CHECK(v < vis[i]);
                ++nsel;
            }
            CHECK(nsel >= 1);
        }
    }
    free(blk);
    orc_topk(s, n_k, vis, NULL, n_q, k_max, idx);
    float *q = randv((size_t)(n_q * H * d_qk)), *K = randv((size_t)(n_k * H_kv * d_qk));
    float *V = sep_v ? randv((size_t)(n_k * H_kv * d_v)) : NULL;
    double *o = malloc((size_t)(n_q * H * d_v) * sizeof(double)), *lse = malloc((size_t)(n_q * H) * sizeof(double));
    orc_attention(q, K, V, idx, k_max, n_q, n_k, H, H_kv, d_qk, d_v, 1.0 / sqrt((double)d_qk), o, lse);
    for (int64_t i = 0; i < n_q * H; ++i) CHECK(isfinite(lse[i]));
    for (int64_t i = 0; i < n_q * H * d_v; ++i) CHECK(isfinite(o[i]));
    /* a row whose selection is all padding: O = 0, LSE = -inf */
    for (int r = 0; r < k_max; ++r) idx[r] = -1;
    orc_attention(q, K, V, idx, k_max, 1, n_k, H, H_kv, d_qk, d_v, 0.125, o, lse);
    for (int h = 0; h < H; ++h) CHECK(isinf(lse[h]) && lse[h] < 0);
    for (int c = 0; c < H * d_v; ++c) CHECK(o[c] == 0.0);
    free(q_i); free(w); free(k_i); free(vis); free(kr); free(s); free(a); free(idx); free(q); free(K); free(V); free(o); free(lse);
    return 0;
}

int main(void)
{
    if (run_case(1, 1, 1, 1, 1, 1, 1, 1, 1, 0)) return 1;      /* one query, one key */
    if (run_case(5, 9, 3, 8, 16, 2, 2, 8, 8, 1)) return 1;     /* k larger than every row */
    if (run_case(17, 40, 4, 32, 6, 4, 1, 24, 16, 0)) return 1; /* latent row: V = first d_v cols */
    if (run_case(9, 70, 2, 16, 20, 8, 2, 32, 32, 1)) return 1; /* grouped kv heads */
    puts("ok");
    return 0;
}
"""


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", str(drv), ORACLE_C, "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert r.stdout.strip() == "ok"
