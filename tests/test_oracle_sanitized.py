"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle's C file is compiled twice with gcc, once plain and once with
-fsanitize=address,undefined (host code only; nothing here touches a GPU),
together with a small driver that runs its entry points on seeded inputs:
every memory depth (linear, 2-layer, 4-layer), both read modes, chunks that
leave a ragged tail, one-token chunks, an empty sequence and the argument
errors.  The sanitized build must finish without a report, and both builds
must print the same outputs bit for bit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "titans_oracle.c")

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t tmo_param_count(int d, int hidden, int n_layers);
int tmo_memory_apply(int d, int hidden, int n_layers, const double* W, const double* x, double* y);
int tmo_memory_grad(int d, int hidden, int n_layers, const double* W, const double* k, const double* v,
                    double* grad, double* loss);
int tmo_forward(int streams, int N, int d, int hidden, int n_layers, int chunk, int read_mode,
                const double* k, const double* v, const double* q, const double* alpha, const double* eta,
                const double* theta, const double* W_in, const double* S_in, double* y, double* W_out,
                double* S_out, double* w_norm, int n_threads);

static uint64_t st = 12345;
static double rnd(void) {   /* 53-bit uniform in [-1, 1) from a 64-bit LCG */
    st = st * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(int64_t n, double lo, double hi) {
    double* a = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (rnd() + 1.0);
    return a;
}
static void dump(const char* tag, const double* a, int64_t n) {
    uint64_t h = 1469598103934665603ULL;   /* FNV-1a over the bits */
    for (int64_t i = 0; i < n; ++i) {
        uint64_t b;
        memcpy(&b, &a[i], 8);
        for (int j = 0; j < 8; ++j) h = (h ^ ((b >> (8 * j)) & 0xff)) * 1099511628211ULL;
    }
    printf("%s %016llx\n", tag, (unsigned long long)h);
}

static void run(int streams, int N, int d, int hidden, int L, int chunk, int rm) {
    const int64_t P = tmo_param_count(d, hidden, L);
    const int64_t T = (int64_t)streams * N;
    double *k = fill(T * d, -0.5, 0.5), *v = fill(T * d, -1, 1), *q = fill(T * d, -0.5, 0.5);
    double *al = fill(T, 0, 0.1), *et = fill(T, 0.8, 1), *th = fill(T, 0, 0.1);
    double *W = fill(streams * P, -0.2, 0.2), *S = fill(streams * P, -0.01, 0.01);
    double *y = fill(T * d, 0, 0), *Wo = fill(streams * P, 0, 0), *So = fill(streams * P, 0, 0);
    const int64_t nc = chunk > 0 ? (N + chunk - 1) / chunk : 1;
    double* wn = fill(streams * nc, 0, 0);
    char tag[96];
    int rc = tmo_forward(streams, N, d, hidden, L, chunk, rm, k, v, q, al, et, th, W, S, y, Wo, So, wn, 2);
    snprintf(tag, sizeof tag, "fwd s%d N%d d%d h%d L%d b%d rm%d rc%d", streams, N, d, hidden, L, chunk, rm, rc);
    printf("%s\n", tag);
    dump(" y", y, T * d);
    dump(" W", Wo, streams * P);
    dump(" S", So, streams * P);
    dump(" wn", wn, streams * nc);
    if (N > 0) {
        double* yo = fill(d, 0, 0);
        double* g = fill(P, 0, 0);
        double loss = 0;
        printf("apply rc%d grad rc%d\n", tmo_memory_apply(d, hidden, L, W, q, yo),
               tmo_memory_grad(d, hidden, L, W, k, v, g, &loss));
        dump(" apply", yo, d);
        dump(" grad", g, P);
        dump(" loss", &loss, 1);
        free(yo);
        free(g);
    }
    free(k); free(v); free(q); free(al); free(et); free(th); free(W); free(S); free(y); free(Wo); free(So); free(wn);
}

int main(void) {
    run(2, 37, 8, 8, 1, 5, 0);
    run(2, 37, 8, 8, 1, 5, 1);
    run(3, 29, 8, 16, 2, 7, 0);
    run(1, 16, 8, 12, 2, 1, 0);
    run(2, 21, 4, 8, 4, 4, 1);
    run(1, 0, 8, 8, 2, 4, 0);
    printf("bad args %d %d\n", tmo_forward(1, 4, 8, 8, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1),
           tmo_forward(1, 4, 8, 8, 2, 4, 7, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1));
    return 0;
}
"""


def _build(tmp, name, extra):
    drv = os.path.join(tmp, "driver.c")
    with open(drv, "w") as fh:
        fh.write(DRIVER)
    exe = os.path.join(tmp, name)
    subprocess.check_call(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-o", exe, drv, SRC, "-lm"] + extra)
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_clean_under_address_and_undefined_sanitizers(tmp_path):
    plain = _build(str(tmp_path), "plain", [])
    sani = _build(str(tmp_path), "sanitized",
                  ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    ref = subprocess.run([plain], capture_output=True, text=True, env=env, timeout=300)
    out = subprocess.run([sani], capture_output=True, text=True, env=env, timeout=300)
    assert ref.returncode == 0, ref.stderr
    assert out.returncode == 0, out.stderr[-4000:]
    assert "runtime error" not in out.stderr and "Sanitizer" not in out.stderr, out.stderr[-4000:]
    assert out.stdout == ref.stdout
    assert "fwd s1 N0" in out.stdout and "bad args -1 -1" in out.stdout
