/*
 * The oracle (oracle/msda_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: seeded problems on tiny and degenerate maps
 * (1x1, 1xW, Hx1), locations far off the map, NaN and +-Inf, one and several
 * OpenMP threads.  Every buffer is allocated at its exact size, so a read or
 * write past a tensor is reported.  Checks that the outputs are finite and
 * that the thread count does not change them.  Prints "oracle_driver ok".
 * Built and run by tests/test_sanitize_host.py (gcc, no GPU).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_forward(int64_t bs, int64_t K, int64_t M, int64_t D, int64_t L, int64_t P, int64_t Q,
                    const int64_t *shapes, const int64_t *starts, const float *value, const float *loc,
                    const double *attw, double *out, int nthreads);
void oracle_backward(int64_t bs, int64_t K, int64_t M, int64_t D, int64_t L, int64_t P, int64_t Q,
                     const int64_t *shapes, const int64_t *starts, const float *value, const float *loc,
                     const double *attw, const float *grad_out, double *grad_value, double *grad_loc,
                     double *grad_w, int nthreads);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint64_t next(void) {                 /* splitmix64 */
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double unif(void) { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "oracle_driver: out of memory\n"); exit(2); }
    return p;
}

static int all_finite(const double *a, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int run_case(int64_t bs, int64_t M, int64_t D, int64_t L, int64_t P, int64_t Q, const int64_t *shapes) {
    int64_t starts[8], K = 0;
    for (int64_t l = 0; l < L; ++l) { starts[l] = K; K += shapes[2 * l] * shapes[2 * l + 1]; }
    const int64_t nv = bs * K * M * D, ns = bs * Q * M * L * P, no = bs * Q * M * D;
    float *value = xmalloc(sizeof(float) * nv), *loc = xmalloc(sizeof(float) * 2 * ns), *g = xmalloc(sizeof(float) * no);
    double *w = xmalloc(sizeof(double) * ns);
    double *out1 = xmalloc(sizeof(double) * no), *out4 = xmalloc(sizeof(double) * no);
    double *gv1 = xmalloc(sizeof(double) * nv), *gl1 = xmalloc(sizeof(double) * 2 * ns), *gw1 = xmalloc(sizeof(double) * ns);
    double *gv4 = xmalloc(sizeof(double) * nv), *gl4 = xmalloc(sizeof(double) * 2 * ns), *gw4 = xmalloc(sizeof(double) * ns);
    for (int64_t i = 0; i < nv; ++i) value[i] = (float)(2.0 * unif() - 1.0);
    for (int64_t i = 0; i < no; ++i) g[i] = (float)(2.0 * unif() - 1.0);
    for (int64_t i = 0; i < ns; ++i) {
        w[i] = unif();
        const uint64_t kind = next() % 16;
        float x = (float)(1.6 * unif() - 0.3), y = (float)(1.6 * unif() - 0.3);
        if (kind == 0) x = NAN;
        else if (kind == 1) y = INFINITY;
        else if (kind == 2) x = -INFINITY;
        else if (kind == 3) { x = 1e30f; y = -1e30f; }
        else if (kind == 4) { x = 0.5f / (float)shapes[2 * ((i / P) % L) + 1]; }     /* a pixel centre */
        loc[2 * i] = x;
        loc[2 * i + 1] = y;
    }
    oracle_forward(bs, K, M, D, L, P, Q, shapes, starts, value, loc, w, out1, 1);
    oracle_forward(bs, K, M, D, L, P, Q, shapes, starts, value, loc, w, out4, 4);
    oracle_backward(bs, K, M, D, L, P, Q, shapes, starts, value, loc, w, g, gv1, gl1, gw1, 1);
    oracle_backward(bs, K, M, D, L, P, Q, shapes, starts, value, loc, w, g, gv4, gl4, gw4, 4);
    int ok = all_finite(out1, no) && all_finite(gv1, nv) && all_finite(gl1, 2 * ns) && all_finite(gw1, ns) &&
             memcmp(out1, out4, sizeof(double) * no) == 0 && memcmp(gl1, gl4, sizeof(double) * 2 * ns) == 0 &&
             memcmp(gw1, gw4, sizeof(double) * ns) == 0 && memcmp(gv1, gv4, sizeof(double) * nv) == 0;
    free(value); free(loc); free(g); free(w); free(out1); free(out4);
    free(gv1); free(gl1); free(gw1); free(gv4); free(gl4); free(gw4);
    return ok;
}

int main(void) {
    static const int64_t maps[][2] = {{1, 1}, {1, 5}, {4, 1}, {3, 5}, {7, 6}, {13, 17}, {2, 64}, {25, 34}};
    const int nmaps = (int)(sizeof maps / sizeof maps[0]);
    int cases = 0;
    for (int it = 0; it < 300; ++it) {
        const int64_t L = 1 + (int64_t)(next() % 4), P = 1 + (int64_t)(next() % 4);
        const int64_t bs = (int64_t)(next() % 3), M = 1 + (int64_t)(next() % 3);
        const int64_t D = 8 * (1 + (int64_t)(next() % 2)), Q = (int64_t)(next() % 9);
        int64_t shapes[8];
        for (int64_t l = 0; l < L; ++l) {
            const int k = (int)(next() % (uint64_t)nmaps);
            shapes[2 * l] = maps[k][0];
            shapes[2 * l + 1] = maps[k][1];
        }
        if (!run_case(bs, M, D, L, P, Q, shapes)) {
            fprintf(stderr, "oracle_driver: case %d (bs %ld M %ld D %ld L %ld P %ld Q %ld) not finite or thread-dependent\n",
                    it, (long)bs, (long)M, (long)D, (long)L, (long)P, (long)Q);
            return 1;
        }
        ++cases;
    }
    printf("oracle_driver ok: %d cases\n", cases);
    return 0;
}
