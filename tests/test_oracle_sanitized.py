"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle.c is compiled together with a small C driver with gcc's address and
undefined-behaviour sanitizers, and the driver walks the oracle's argument
space: dense and packed layouts (empty, one-token and ragged sequences),
causal and not, key ranges (empty, clipped, past the end), more threads than
rows, and the invalid-argument and invalid-row returns.  Any out-of-bounds
access, leak, overflow or other undefined behaviour aborts the driver with a
sanitizer report; the driver also checks that every visible row's weights
reproduce its LSE.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_rows_range(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                int B, int H, int N, int d, float scale, int causal,
                                const int32_t *cu_seqlens, int64_t n_rows, const int64_t *rows,
                                int kv_lo, int kv_hi, double *o_out, double *lse_out, int nthreads);
int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int B, int H, int N, int d, float scale, int causal,
                          const int32_t *cu_seqlens, int64_t n_rows, const int64_t *rows,
                          double *o_out, double *lse_out, int nthreads);

static uint32_t state = 12345u;
static uint16_t rnd_bf16(void) {
    state = state * 1664525u + 1013904223u;
    float x = ((float)(state >> 8) / 16777216.0f - 0.5f) * 4.0f;
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}
static double widen(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int fails = 0;

/* every row of one layout; checks sum_j exp(s_ij - lse_i) = 1 over the visible keys */
static void run(int B, int H, int d, const int32_t *cu, int N, int causal, int lo, int hi, int threads) {
    int64_t T = cu ? cu[B] : (int64_t)B * N;
    size_t elems = (size_t)T * H * d;
    uint16_t *q = malloc(elems * 2 + 2), *k = malloc(elems * 2 + 2), *v = malloc(elems * 2 + 2);
    for (size_t i = 0; i < elems; ++i) { q[i] = rnd_bf16(); k[i] = rnd_bf16(); v[i] = rnd_bf16(); }
    int64_t nrows = 0;
    int64_t *rows = malloc(sizeof(int64_t) * 3 * (T * H + 1));
    for (int b = 0; b < B; ++b) {
        int n = cu ? cu[b + 1] - cu[b] : N;
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < n; ++i) { rows[3 * nrows] = b; rows[3 * nrows + 1] = h; rows[3 * nrows + 2] = i; ++nrows; }
    }
    double *o = malloc(sizeof(double) * (size_t)(nrows * d + 1)), *lse = malloc(sizeof(double) * (size_t)(nrows + 1));
    float scale = 1.0f / sqrtf((float)d);
    int rc = oracle_attention_rows_range(q, k, v, B, H, N, d, scale, causal, cu, nrows, rows, lo, hi, o, lse, threads);
    if (rc != 0) { printf("rc %d\n", rc); ++fails; }
    for (int64_t r = 0; r < nrows; ++r) {
        int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
        int64_t t0 = cu ? cu[b] : (int64_t)b * N;
        int n = cu ? cu[b + 1] - cu[b] : N;
        int jend = causal ? (i + 1 < n ? i + 1 : n) : n;
        int j0 = lo > 0 ? lo : 0, j1 = hi < jend ? hi : jend;
        if (j1 <= j0) {
            if (!(isinf(lse[r]) && lse[r] < 0)) { printf("empty row lse %g\n", lse[r]); ++fails; }
            continue;
        }
        double tot = 0.0;
        for (int j = j0; j < j1; ++j) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += widen(q[((t0 + i) * H + h) * d + c]) * widen(k[((t0 + j) * H + h) * d + c]);
            tot += exp(s * (double)scale - lse[r]);
        }
        if (fabs(tot - 1.0) > 1e-9) { printf("row weights sum %g\n", tot); ++fails; }
    }
    free(q); free(k); free(v); free(rows); free(o); free(lse);
}

int main(void) {
    run(2, 3, 8, NULL, 17, 0, 0, 17, 4);
    run(2, 3, 8, NULL, 17, 1, 0, 17, 64);     /* more threads than rows */
    run(1, 2, 16, NULL, 33, 1, 5, 20, 3);     /* key range inside */
    run(1, 2, 16, NULL, 33, 0, 30, 99, 2);    /* range past the end */
    run(1, 1, 8, NULL, 9, 1, 4, 4, 2);        /* empty range */
    int32_t cu[] = {0, 0, 1, 6, 6, 19};       /* empty, one-token and ragged sequences */
    run(5, 2, 8, cu, 13, 0, 0, 13, 3);
    run(5, 2, 8, cu, 13, 1, 0, 13, 3);
    run(5, 2, 8, cu, 13, 1, 2, 7, 8);
    /* invalid arguments and rows return an error code and touch nothing */
    uint16_t x[64] = {0};
    int64_t bad[3] = {0, 0, 9};
    double o[8], l[1];
    if (oracle_attention_rows(x, x, x, 1, 1, 4, 8, 1.0f, 0, NULL, 1, bad, o, l, 1) == 0) { puts("row past n accepted"); ++fails; }
    if (oracle_attention_rows(NULL, x, x, 1, 1, 4, 8, 1.0f, 0, NULL, 1, bad, o, l, 1) == 0) { puts("NULL accepted"); ++fails; }
    if (oracle_attention_rows(x, x, x, 0, 1, 4, 8, 1.0f, 0, NULL, 1, bad, o, l, 1) == 0) { puts("B = 0 accepted"); ++fails; }
    printf("failures %d\n", fails);
    return fails != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_asan"
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         SRC, str(drv), "-o", str(exe), "-lm"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "failures 0" in res.stdout
