/*
 * oracle_driver.c -- runs every function of the fp64 C oracle on small ragged
 * problems under AddressSanitizer and UndefinedBehaviorSanitizer (host-only
 * build, see tests/test_sanitizers.py).  Every buffer is allocated at its exact
 * size, so an index one past an end is reported.  The functions are also
 * checked against each other, so the run exercises the real code paths:
 *   - L single steps reproduce the forward (y and final state);
 *   - state passing over the chunk-local states gives the forward's chunk-start
 *     states and final state; the chunk scan from them gives the forward's y;
 *   - the cumulative sum's last entry of each chunk is log2(e) * sum dt*A.
 * Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ssd_oracle_forward(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double* x,
                       const double* dt, const double* dt_in, const double* A, const double* B, const double* C,
                       const double* D, const double* h0, double* y, double* final_state, int64_t chunk,
                       double* chunk_start, double* chunk_local, int nthreads);
int ssd_oracle_step(int64_t b, int64_t H, int64_t P, int64_t N, int64_t G, double* state, const double* x,
                    const double* dt, const double* dt_in, const double* A, const double* B, const double* C,
                    const double* D, double* y, int nthreads);
int ssd_oracle_dt_frontend(int64_t n, int64_t H, const double* raw, const double* A, const double* bias,
                           int softplus, int zoh, int clamp, double lo, double hi, double* dt_decay,
                           double* dt_input);
int ssd_oracle_chunk_cumsum(int64_t b, int64_t L, int64_t H, int64_t Q, const double* dt, const double* dt_in,
                            const double* A, double* dt_t, double* cs_log2);
int ssd_oracle_state_passing(int64_t b, int64_t nC, int64_t H, int64_t P, int64_t N, int64_t Q,
                             const double* local, const double* cs_log2, const double* h0, double* chunk_start,
                             double* final_state);
int ssd_oracle_chunk_scan(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q,
                          const double* x, const double* dt, const double* A, const double* B, const double* C,
                          const double* D, const double* chunk_start, double* y, int nthreads);
int ssd_oracle_selective_scan(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G, const double* x,
                              const double* delta, const double* A, const double* B, const double* C,
                              const double* Dskip, const double* h0, double* y, double* final_state, int zoh,
                              int nthreads);
int ssd_oracle_backward(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double* x,
                        const double* dt, const double* A, const double* B, const double* C, const double* D,
                        const double* h0, const double* dy, const double* dfinal, double* dx, double* ddt,
                        double* dA, double* dB, double* dC, double* dD, double* dh0, int nthreads);

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [0, 1) */
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return (double)((g_rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static double* vec(size_t n, double lo, double hi) {
    double* p = (double*)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}
static double* zeros(size_t n) { return (double*)calloc(n ? n : 1, sizeof(double)); }
static double maxdiff(const double* a, const double* b, size_t n) {
    double m = 0.0;
    for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}
static int fails = 0;
static void expect(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++fails;
    }
}

static void ssd_case(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q) {
    const size_t nx = (size_t)(b * L * H * P), ndt = (size_t)(b * L * H), nbc = (size_t)(b * L * G * N),
                 ns = (size_t)(b * H * P * N);
    const int64_t nC = (L + Q - 1) / Q;
    const size_t nst = (size_t)(b * nC * H * P * N), ncs = (size_t)(b * H * nC * Q);
    double *x = vec(nx, -1, 1), *dt = vec(ndt, 1e-3, 0.2), *A = vec((size_t)H, -4, -0.5);
    double *B = vec(nbc, -0.3, 0.3), *C = vec(nbc, -0.3, 0.3), *D = vec((size_t)H, -1, 1), *h0 = vec(ns, -0.1, 0.1);
    double *y = zeros(nx), *fin = zeros(ns), *cstart = zeros(nst), *clocal = zeros(nst);
    expect(ssd_oracle_forward(b, L, H, P, N, G, x, dt, NULL, A, B, C, D, h0, y, fin, Q, cstart, clocal, 1) == 0,
           "forward");
    /* single steps */
    double *S = zeros(ns), *ys = zeros(nx), *xt = zeros((size_t)(b * H * P)), *dtt = zeros((size_t)(b * H));
    double *Bt = zeros((size_t)(b * G * N)), *Ct = zeros((size_t)(b * G * N)), *yt = zeros((size_t)(b * H * P));
    memcpy(S, h0, ns * sizeof(double));
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t bb = 0; bb < b; ++bb) {
            memcpy(xt + bb * H * P, x + (bb * L + t) * H * P, (size_t)(H * P) * sizeof(double));
            memcpy(dtt + bb * H, dt + (bb * L + t) * H, (size_t)H * sizeof(double));
            memcpy(Bt + bb * G * N, B + (bb * L + t) * G * N, (size_t)(G * N) * sizeof(double));
            memcpy(Ct + bb * G * N, C + (bb * L + t) * G * N, (size_t)(G * N) * sizeof(double));
        }
        expect(ssd_oracle_step(b, H, P, N, G, S, xt, dtt, NULL, A, Bt, Ct, D, yt, 1) == 0, "step");
        for (int64_t bb = 0; bb < b; ++bb)
            memcpy(ys + (bb * L + t) * H * P, yt + bb * H * P, (size_t)(H * P) * sizeof(double));
    }
    expect(maxdiff(ys, y, nx) < 1e-12, "steps == forward (y)");
    expect(maxdiff(S, fin, ns) < 1e-12, "steps == forward (final)");
    /* staged calls */
    double *dt_t = zeros(ncs), *cs = zeros(ncs), *start2 = zeros(nst), *fin2 = zeros(ns), *y2 = zeros(nx);
    expect(ssd_oracle_chunk_cumsum(b, L, H, Q, dt, NULL, A, dt_t, cs) == 0, "chunk_cumsum");
    for (int64_t h = 0; h < H && L > 0; ++h) {
        double run = 0.0;
        for (int64_t t = 0; t < (L < Q ? L : Q); ++t) run += dt[t * H + h] * A[h];
        expect(fabs(cs[(h * nC + 0) * Q + Q - 1] - run * 1.4426950408889634) < 1e-12, "cumsum chunk total");
    }
    expect(ssd_oracle_state_passing(b, nC, H, P, N, Q, clocal, cs, h0, start2, fin2) == 0, "state_passing");
    expect(maxdiff(start2, cstart, nst) < 1e-12, "state passing == forward chunk starts");
    expect(maxdiff(fin2, fin, ns) < 1e-12, "state passing == forward final");
    expect(ssd_oracle_chunk_scan(b, L, H, P, N, G, Q, x, dt, A, B, C, D, start2, y2, 1) == 0, "chunk_scan");
    expect(maxdiff(y2, y, nx) < 1e-12, "chunk scan == forward y");
    /* front-end and backward */
    double *dec = zeros(ndt), *inp = zeros(ndt), *bias = vec((size_t)H, -1, 1);
    expect(ssd_oracle_dt_frontend((int64_t)(b * L), H, dt, A, bias, 1, 1, 1, 1e-3, 0.5, dec, inp) == 0,
           "dt_frontend");
    double *dy = vec(nx, -1, 1), *dfin = vec(ns, -1, 1), *dx = zeros(nx), *ddt = zeros(ndt), *dA = zeros((size_t)H);
    double *dB = zeros(nbc), *dC = zeros(nbc), *dD = zeros((size_t)H), *dh0 = zeros(ns);
    expect(ssd_oracle_backward(b, L, H, P, N, G, x, dt, A, B, C, D, h0, dy, dfin, dx, ddt, dA, dB, dC, dD, dh0, 1) ==
               0,
           "backward");
    double* all[] = {x, dt, A, B, C, D, h0, y, fin, cstart, clocal, S, ys, xt, dtt, Bt, Ct, yt, dt_t, cs, start2,
                     fin2, y2, dec, inp, bias, dy, dfin, dx, ddt, dA, dB, dC, dD, dh0};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
}

static void selective_case(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G) {
    const size_t nx = (size_t)(b * L * Dc), nbc = (size_t)(b * L * G * N), ns = (size_t)(b * Dc * N);
    double *x = vec(nx, -1, 1), *dl = vec(nx, 1e-3, 0.2), *A = vec((size_t)(Dc * N), -4, -0.5);
    double *B = vec(nbc, -1, 1), *C = vec(nbc, -1, 1), *D = vec((size_t)Dc, -1, 1), *h0 = vec(ns, -1, 1);
    double *y = zeros(nx), *fin = zeros(ns), *y1 = zeros(nx), *fin1 = zeros(ns);
    expect(ssd_oracle_selective_scan(b, L, Dc, N, G, x, dl, A, B, C, D, h0, y, fin, 1, 1) == 0, "selective zoh");
    expect(ssd_oracle_selective_scan(b, L, Dc, N, G, x, dl, A, B, C, NULL, NULL, y1, fin1, 0, 1) == 0,
           "selective dB");
    double* all[] = {x, dl, A, B, C, D, h0, y, fin, y1, fin1};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
}

int main(void) {
    ssd_case(2, 37, 4, 3, 5, 2, 8);   /* ragged last chunk, two groups */
    ssd_case(1, 64, 2, 4, 4, 1, 16);  /* chunk-aligned */
    ssd_case(1, 1, 3, 2, 3, 3, 4);    /* one token */
    ssd_case(1, 70, 1, 2, 2, 1, 70);  /* one chunk (backward crosses its 64-token blocks) */
    selective_case(2, 29, 6, 5, 3);
    selective_case(1, 1, 4, 3, 1);
    /* rejected arguments return -1 without touching memory */
    expect(ssd_oracle_forward(1, 4, 3, 2, 2, 2, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL,
                              NULL, 1) == -1,
           "H % G rejected");
    if (fails) return 1;
    printf("oracle driver: all checks passed\n");
    return 0;
}
