/*
 * ssd_oracle.c -- plain fp64 CPU oracle for the Mamba-2 selective state-space
 * recurrence and for each staged call of the chunked (SSD) forward.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code with the HIP library
 * and is never on the product path.
 *
 * What is computed (per batch row b and head h, group g = h / (H / G)):
 *
 *   S <- h0[b,h] (or 0)                                 P x N state
 *   for t = 0 .. L-1:
 *       a      = exp(dt[b,t,h] * A[h])                  discretised decay
 *       S[p,n] = a * S[p,n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *       y[b,t,h,p] = sum_n C[b,t,g,n] * S[p,n] + D[h] * x[b,t,h,p]
 *   final[b,h] = S
 *
 * Sources: the discretisation abar = exp(delta * A) is written out in
 * "3.3 Hardware-Aware algorithms and GPU memory hierarchy optimisation",
 * section 2.1; the first-order recurrence h_t = abar_t h_{t-1} + bbar_t x_t and
 * its output through C in the same chapter, sections 3 and 4.1.  Mamba-2 uses
 * one scalar A per head and the input matrix bbar = dt * B (not the
 * zero-order-hold form of section 2.1); the output is read after the update.
 * The staged calls (in-chunk cumulative sum kept in log2 units, chunk states,
 * chunk-order state passing, chunk output from the chunk-start state) follow
 * the three-kernel description on the devotd.net page on the NVIDIA / Jane
 * Street cuTile Mamba-2 forward kernels, section 2.  Each staged call here is
 * written as the plain definition of its result (a token recurrence over the
 * chunk), not as the chunked algebra.
 *
 * Optional dt front-end (ssd_oracle_dt_frontend): a per-head bias, softplus
 * and a clamp turn a raw dt into the step; the zero-order-hold (ZOH) input
 * matrix of "3.3 Hardware-Aware ..." section 2.1 replaces dt in the input term
 * by (exp(dt A) - 1) / A (for scalar A the ZOH B-bar is that factor times B).
 * Every recurrence below therefore takes the decay step dt and, optionally, a
 * separate input step dt_in (NULL: the input term uses dt).
 *
 * Layouts (row-major, contiguous): x, y (b,L,H,P); dt (b,L,H); A, D (H);
 * B, C (b,L,G,N); h0, final, step state (b,H,P,N); per-chunk states
 * (b,nC,H,P,N); dt_t and the log2 cumulative sum (b,H,nC,Q).
 *
 * Built with -O2 -ffp-contract=off and no fast-math; threads split the
 * independent (b, h) slices.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LOG2E_D 1.4426950408889634073599246810019

int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* One token of the recurrence for one (b, h): S <- a*S + dtu*x (outer) B with
 * a = exp(dt*A), then y = C.S + D*x.  dt is the decay step and dtu the input
 * step (equal unless a front-end says otherwise).  Pointers are already offset
 * to this token and head. */
static void token_update(int64_t P, int64_t N, double* S, double dt, double dtu, double A,
                         const double* x, const double* B, const double* C,
                         double Dh, int has_D, double* y) {
    double a = exp(dt * A);
    for (int64_t p = 0; p < P; ++p) {
        double u = dtu * x[p];
        double* row = S + p * N;
        for (int64_t n = 0; n < N; ++n) row[n] = a * row[n] + u * B[n];
    }
    if (y == NULL) return;
    for (int64_t p = 0; p < P; ++p) {
        const double* row = S + p * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += C[n] * row[n];
        y[p] = acc + (has_D ? Dh * x[p] : 0.0);
    }
}

static int bad_dims(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G) {
    return b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || (H % G) != 0;
}

/*
 * Full forward by the token recurrence.  Optional outputs (NULL to skip):
 *   chunk_start  (b,nC,H,P,N): the state before token c*chunk, i.e. after
 *                the first c*chunk tokens (h0 for c = 0);
 *   chunk_local  (b,nC,H,P,N): the state the tokens of chunk c alone produce
 *                from a zero start.
 * Returns 0, or -1 on inconsistent arguments.
 */
int ssd_oracle_forward(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                       const double* x, const double* dt, const double* dt_in, const double* A,
                       const double* B, const double* C, const double* D,
                       const double* h0, double* y, double* final_state,
                       int64_t chunk, double* chunk_start, double* chunk_local,
                       int nthreads) {
    if (bad_dims(b, L, H, P, N, G)) return -1;
    if ((chunk_start || chunk_local) && chunk <= 0) return -1;
    int64_t nC = chunk > 0 ? (L + chunk - 1) / chunk : 0;
    int64_t hpg = H / G;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < b * H; ++bh) {
        int64_t bb = bh / H, h = bh % H, g = h / hpg;
        double* S = (double*)calloc((size_t)(P * N), sizeof(double));
        if (!S) { err = 1; continue; }
        if (h0) memcpy(S, h0 + bh * P * N, sizeof(double) * P * N);
        for (int64_t t = 0; t < L; ++t) {
            if (chunk_start && t % chunk == 0)
                memcpy(chunk_start + ((bb * nC + t / chunk) * H + h) * P * N, S, sizeof(double) * P * N);
            int64_t bt = bb * L + t;
            token_update(P, N, S, dt[bt * H + h], (dt_in ? dt_in : dt)[bt * H + h], A[h],
                         x + (bt * H + h) * P, B + (bt * G + g) * N, C + (bt * G + g) * N,
                         D ? D[h] : 0.0, D != NULL, y ? y + (bt * H + h) * P : NULL);
        }
        if (final_state) memcpy(final_state + bh * P * N, S, sizeof(double) * P * N);
        if (chunk_local) {
            for (int64_t c = 0; c < nC; ++c) {
                memset(S, 0, sizeof(double) * P * N);
                int64_t t1 = (c + 1) * chunk < L ? (c + 1) * chunk : L;
                for (int64_t t = c * chunk; t < t1; ++t) {
                    int64_t bt = bb * L + t;
                    token_update(P, N, S, dt[bt * H + h], (dt_in ? dt_in : dt)[bt * H + h], A[h],
                                 x + (bt * H + h) * P, B + (bt * G + g) * N, C + (bt * G + g) * N, 0.0, 0,
                                 NULL);
                }
                memcpy(chunk_local + ((bb * nC + c) * H + h) * P * N, S, sizeof(double) * P * N);
            }
        }
        free(S);
    }
    return err ? -2 : 0;
}

/*
 * One decode step for every (b, h): the O(1) fixed-size state update of the
 * "Compiler-First State Space Duality and Portable O(1) Autoregressive Caching
 * for Inference" summary (Methodology, on-device O(1) caching).  state is
 * (b,H,P,N), updated in place; x (b,H,P); dt (b,H); B, C (b,G,N); y (b,H,P).
 */
int ssd_oracle_step(int64_t b, int64_t H, int64_t P, int64_t N, int64_t G,
                    double* state, const double* x, const double* dt, const double* dt_in, const double* A,
                    const double* B, const double* C, const double* D, double* y,
                    int nthreads) {
    if (bad_dims(b, 1, H, P, N, G)) return -1;
    int64_t hpg = H / G;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < b * H; ++bh) {
        int64_t bb = bh / H, h = bh % H, g = h / hpg;
        token_update(P, N, state + bh * P * N, dt[bh], (dt_in ? dt_in : dt)[bh], A[h], x + bh * P,
                     B + (bb * G + g) * N, C + (bb * G + g) * N,
                     D ? D[h] : 0.0, D != NULL, y + bh * P);
    }
    return 0;
}

/*
 * dt front-end, elementwise over n rows of H heads (row-major (n, H)):
 *   d = raw + bias[h]                       (bias may be NULL)
 *   d = softplus(d) = log(1 + exp(d))       if softplus
 *   d = min(max(d, lo), hi)                 if clamp
 *   dt_decay = d
 *   dt_input = (exp(d A) - 1) / A           if zoh (A != 0; d when A == 0)
 *            = d                            otherwise
 * The ZOH factor is the scalar-A form of the zero-order-hold B-bar of
 * "3.3 Hardware-Aware ..." section 2.1: integrating S' = A S + B x over a step
 * of length d with x held constant gives exp(dA) S + (exp(dA) - 1)/A B x.
 */
int ssd_oracle_dt_frontend(int64_t n, int64_t H, const double* raw, const double* A, const double* bias,
                           int softplus, int zoh, int clamp, double lo, double hi,
                           double* dt_decay, double* dt_input) {
    if (n < 0 || H <= 0) return -1;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t h = 0; h < H; ++h) {
            double d = raw[r * H + h];
            if (bias) d = d + bias[h];
            if (softplus) d = d > 0.0 ? d + log1p(exp(-d)) : log1p(exp(d));
            if (clamp) d = d < lo ? lo : (d > hi ? hi : d);
            dt_decay[r * H + h] = d;
            double in = d;
            if (zoh && A[h] != 0.0) in = expm1(d * A[h]) / A[h];
            dt_input[r * H + h] = in;
        }
    return 0;
}

/*
 * In-chunk cumulative sum (devotd.net cuTile page, section 2, first kernel):
 * for chunk c and in-chunk position i, cs_log2 = log2(e) * sum_{k<=i} dt*A over
 * the chunk's tokens; positions past L count as dt = 0.  dt_t receives the
 * input step: dt itself, or dt_in when given (0 past L).  Both outputs are
 * (b,H,nC,Q).
 */
int ssd_oracle_chunk_cumsum(int64_t b, int64_t L, int64_t H, int64_t Q,
                            const double* dt, const double* dt_in, const double* A,
                            double* dt_t, double* cs_log2) {
    if (b < 0 || L < 0 || H <= 0 || Q <= 0) return -1;
    int64_t nC = (L + Q - 1) / Q;
    for (int64_t bb = 0; bb < b; ++bb)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t c = 0; c < nC; ++c) {
                double run = 0.0;
                for (int64_t i = 0; i < Q; ++i) {
                    int64_t t = c * Q + i;
                    double d = t < L ? dt[(bb * L + t) * H + h] : 0.0;
                    run += d * A[h];
                    int64_t o = ((bb * H + h) * nC + c) * Q + i;
                    cs_log2[o] = run * LOG2E_D;
                    if (dt_t) dt_t[o] = t < L && dt_in ? dt_in[(bb * L + t) * H + h] : d;
                }
            }
    return 0;
}

/*
 * Chunk-order state passing (devotd.net cuTile page, section 2, second
 * kernel; associativity of the recurrence, "3.3 Hardware-Aware ..." section
 * 4.1): S_0 = h0 (or 0), chunk_start[c] = S_c, S_{c+1} = 2^{cs_log2[c,Q-1]} S_c
 * + local[c], final = S_nC.  local and chunk_start are (b,nC,H,P,N) and may be
 * the same buffer.
 */
int ssd_oracle_state_passing(int64_t b, int64_t nC, int64_t H, int64_t P, int64_t N, int64_t Q,
                             const double* local, const double* cs_log2, const double* h0,
                             double* chunk_start, double* final_state) {
    if (b < 0 || nC < 0 || H <= 0 || P <= 0 || N <= 0 || Q <= 0) return -1;
    int64_t PN = P * N;
    double* S = (double*)malloc(sizeof(double) * (size_t)PN);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)PN);
    if (!S || !tmp) { free(S); free(tmp); return -2; }
    for (int64_t bb = 0; bb < b; ++bb)
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t e = 0; e < PN; ++e) S[e] = h0 ? h0[(bb * H + h) * PN + e] : 0.0;
            for (int64_t c = 0; c < nC; ++c) {
                int64_t o = ((bb * nC + c) * H + h) * PN;
                double decay = exp2(cs_log2[((bb * H + h) * nC + c) * Q + (Q - 1)]);
                memcpy(tmp, local + o, sizeof(double) * PN);
                if (chunk_start) memcpy(chunk_start + o, S, sizeof(double) * PN);
                for (int64_t e = 0; e < PN; ++e) S[e] = decay * S[e] + tmp[e];
            }
            if (final_state) memcpy(final_state + (bb * H + h) * PN, S, sizeof(double) * PN);
        }
    free(S);
    free(tmp);
    return 0;
}

/*
 * Chunk output from the chunk-start state (devotd.net cuTile page, section 2,
 * third kernel): for every chunk c, run the token recurrence over the chunk's
 * tokens starting from chunk_start[c] and emit y.  chunk_start is
 * (b,nC,H,P,N) with nC = ceil(L/Q).
 */
int ssd_oracle_chunk_scan(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q,
                          const double* x, const double* dt, const double* A,
                          const double* B, const double* C, const double* D,
                          const double* chunk_start, double* y, int nthreads) {
    if (bad_dims(b, L, H, P, N, G) || Q <= 0) return -1;
    int64_t nC = (L + Q - 1) / Q, hpg = H / G;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t w = 0; w < b * nC * H; ++w) {
        int64_t bb = w / (nC * H), c = (w / H) % nC, h = w % H, g = h / hpg;
        double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));
        if (!S) { err = 1; continue; }
        memcpy(S, chunk_start + w * P * N, sizeof(double) * P * N);
        int64_t t1 = (c + 1) * Q < L ? (c + 1) * Q : L;
        for (int64_t t = c * Q; t < t1; ++t) {
            int64_t bt = bb * L + t;
            token_update(P, N, S, dt[bt * H + h], dt[bt * H + h], A[h], x + (bt * H + h) * P,
                         B + (bt * G + g) * N, C + (bt * G + g) * N,
                         D ? D[h] : 0.0, D != NULL, y + (bt * H + h) * P);
        }
        free(S);
    }
    return err ? -2 : 0;
}

/*
 * Mamba-1 selective scan (the per-channel selective SSM of "3.3 Hardware-Aware
 * algorithms and GPU memory hierarchy optimisation", sections 2.1 and 3): for
 * every batch row b and channel d (group g = d / (Dc / G)), with a diagonal
 * state of N entries and a per-entry A[d,n]:
 *
 *   h <- h0[b,d] (or 0)
 *   for t = 0 .. L-1:
 *       abar[n] = exp(delta[b,t,d] * A[d,n])
 *       bbar[n] = (exp(delta A[d,n]) - 1) / A[d,n] * B[b,t,g,n]   zero-order hold (zoh != 0;
 *                                                                 delta * B when A[d,n] == 0)
 *               = delta[b,t,d] * B[b,t,g,n]                        otherwise
 *       h[n] = abar[n] * h[n] + bbar[n] * x[b,t,d]
 *       y[b,t,d] = sum_n C[b,t,g,n] * h[n] + Dskip[d] * x[b,t,d]
 *   final[b,d] = h
 *
 * delta is the step after any front-end (bias, softplus, clamp).  Layouts:
 * x, delta, y (b,L,Dc); A (Dc,N); B, C (b,L,G,N); Dskip (Dc); h0, final
 * (b,Dc,N).  Threads split the independent (b, d) rows.
 */
int ssd_oracle_selective_scan(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G,
                              const double* x, const double* delta, const double* A,
                              const double* B, const double* C, const double* Dskip,
                              const double* h0, double* y, double* final_state, int zoh,
                              int nthreads) {
    if (b < 0 || L < 0 || Dc <= 0 || N <= 0 || G <= 0 || (Dc % G) != 0) return -1;
    int64_t cpg = Dc / G;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bd = 0; bd < b * Dc; ++bd) {
        int64_t bb = bd / Dc, d = bd % Dc, g = d / cpg;
        double* h = (double*)calloc((size_t)N, sizeof(double));
        if (!h) { err = 1; continue; }
        if (h0) memcpy(h, h0 + bd * N, sizeof(double) * N);
        const double* Ad = A + d * N;
        for (int64_t t = 0; t < L; ++t) {
            int64_t bt = bb * L + t;
            double dl = delta[bt * Dc + d], xv = x[bt * Dc + d];
            const double* Bt = B + (bt * G + g) * N;
            const double* Ct = C + (bt * G + g) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double abar = exp(dl * Ad[n]);
                double bbar = dl * Bt[n];
                if (zoh && Ad[n] != 0.0) bbar = expm1(dl * Ad[n]) / Ad[n] * Bt[n];
                h[n] = abar * h[n] + bbar * xv;
                acc += Ct[n] * h[n];
            }
            if (y) y[bt * Dc + d] = acc + (Dskip ? Dskip[d] * xv : 0.0);
        }
        if (final_state) memcpy(final_state + bd * N, h, sizeof(double) * N);
        free(h);
    }
    return err ? -2 : 0;
}

/*
 * Backward pass of the SSD recurrence (reverse-mode derivative of the token
 * recurrence ssd_oracle_forward computes, plain input step dt, no front-end):
 * given dy (b,L,H,P) and the gradient of the final state dfinal (b,H,P,N, may
 * be NULL = 0), returns dx (b,L,H,P), ddt (b,L,H), dA (H), dB, dC (b,L,G,N),
 * dD (H, may be NULL) and dh0 (b,H,P,N, may be NULL).  The training use and
 * the recomputation of forward states instead of storing them follow
 * "3.3 Hardware-Aware ..." section 6.
 *
 * With G_t the gradient with respect to the state after token t, in reverse
 * token order (a_t = exp(dt_t A), S_{-1} = h0):
 *   G <- dfinal (or 0)
 *   for t = L-1 .. 0:
 *       G      += dy_t (outer) C_t                 (y_t = C_t . S_t + D x_t)
 *       dC_t   += S_t^T dy_t                       (summed over the heads of the group)
 *       dx_t    = dt_t G B_t + D dy_t
 *       dB_t   += dt_t G^T x_t                     (summed over the heads of the group)
 *       ddt_t   = sum_{p,n} G (x_t (outer) B_t + A a_t S_{t-1})
 *       dA     += sum_{p,n} G dt_t a_t S_{t-1}
 *       dD     += dy_t . x_t
 *       G      <- a_t G                            (gradient w.r.t. S_{t-1})
 *   dh0 = G
 * The states S_t are recomputed from checkpoints every 64 tokens.  Per-head
 * dB, dC contributions go to a (b,L,H,N) scratch and are summed over heads.
 */
#define BWD_BLOCK 64
int ssd_oracle_backward(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double* x, const double* dt, const double* A, const double* B,
                        const double* C, const double* D, const double* h0, const double* dy,
                        const double* dfinal, double* dx, double* ddt, double* dA, double* dB,
                        double* dC, double* dD, double* dh0, int nthreads) {
    if (bad_dims(b, L, H, P, N, G)) return -1;
    int64_t hpg = H / G, PN = P * N, nblk = (L + BWD_BLOCK - 1) / BWD_BLOCK;
    double* dBh = (double*)calloc((size_t)(b * L * H * N) + 1, sizeof(double));
    double* dCh = (double*)calloc((size_t)(b * L * H * N) + 1, sizeof(double));
    double* dAbh = (double*)calloc((size_t)(b * H) + 1, sizeof(double));
    double* dDbh = (double*)calloc((size_t)(b * H) + 1, sizeof(double));
    if (!dBh || !dCh || !dAbh || !dDbh) { free(dBh); free(dCh); free(dAbh); free(dDbh); return -2; }
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < b * H; ++bh) {
        int64_t bb = bh / H, h = bh % H, g = h / hpg;
        double* ck = (double*)malloc(sizeof(double) * (size_t)((nblk + 1) * PN));
        double* blk = (double*)malloc(sizeof(double) * (size_t)((BWD_BLOCK + 1) * PN));
        double* Gs = (double*)malloc(sizeof(double) * (size_t)PN);
        if (!ck || !blk || !Gs) { err = 1; free(ck); free(blk); free(Gs); continue; }
        /* forward: checkpoint the state before every block */
        double* S = blk;
        for (int64_t e = 0; e < PN; ++e) S[e] = h0 ? h0[bh * PN + e] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            if (t % BWD_BLOCK == 0) memcpy(ck + (t / BWD_BLOCK) * PN, S, sizeof(double) * PN);
            int64_t bt = bb * L + t;
            token_update(P, N, S, dt[bt * H + h], dt[bt * H + h], A[h], x + (bt * H + h) * P,
                         B + (bt * G + g) * N, C + (bt * G + g) * N, 0.0, 0, NULL);
        }
        /* backward over the blocks, last first */
        for (int64_t e = 0; e < PN; ++e) Gs[e] = dfinal ? dfinal[bh * PN + e] : 0.0;
        double dAacc = 0.0, dDacc = 0.0;
        for (int64_t k = nblk - 1; k >= 0; --k) {
            int64_t t0 = k * BWD_BLOCK, t1 = (t0 + BWD_BLOCK < L) ? t0 + BWD_BLOCK : L;
            /* blk[i] = state before token t0 + i; blk[t1 - t0] = state after the block */
            memcpy(blk, ck + k * PN, sizeof(double) * PN);
            for (int64_t t = t0; t < t1; ++t) {
                int64_t bt = bb * L + t;
                double* nxt = blk + (t - t0 + 1) * PN;
                memcpy(nxt, blk + (t - t0) * PN, sizeof(double) * PN);
                token_update(P, N, nxt, dt[bt * H + h], dt[bt * H + h], A[h], x + (bt * H + h) * P,
                             B + (bt * G + g) * N, C + (bt * G + g) * N, 0.0, 0, NULL);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                int64_t bt = bb * L + t;
                const double* xt = x + (bt * H + h) * P;
                const double* dyt = dy + (bt * H + h) * P;
                const double* Bt = B + (bt * G + g) * N;
                const double* Ct = C + (bt * G + g) * N;
                const double* Sprev = blk + (t - t0) * PN;
                const double* Scur = blk + (t - t0 + 1) * PN;
                double d = dt[bt * H + h], a = exp(d * A[h]);
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) Gs[p * N + n] += dyt[p] * Ct[n];
                double* dCt = dCh + (bt * H + h) * N;
                double* dBt = dBh + (bt * H + h) * N;
                for (int64_t n = 0; n < N; ++n) {
                    double sc = 0.0, sb = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        sc += Scur[p * N + n] * dyt[p];
                        sb += Gs[p * N + n] * xt[p];
                    }
                    dCt[n] = sc;
                    dBt[n] = d * sb;
                }
                double dd = 0.0, gs = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    double gb = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        gb += Gs[p * N + n] * Bt[n];
                        gs += Gs[p * N + n] * Sprev[p * N + n];
                    }
                    dx[(bt * H + h) * P + p] = d * gb + (D ? D[h] * dyt[p] : 0.0);
                    dd += gb * xt[p];
                    dDacc += dyt[p] * xt[p];
                }
                ddt[bt * H + h] = dd + A[h] * a * gs;
                dAacc += d * a * gs;
                for (int64_t e = 0; e < PN; ++e) Gs[e] *= a;
            }
        }
        if (dh0) memcpy(dh0 + bh * PN, Gs, sizeof(double) * PN);
        dAbh[bh] = dAacc;
        dDbh[bh] = dDacc;
        free(ck);
        free(blk);
        free(Gs);
    }
    if (!err) {
        for (int64_t h = 0; h < H; ++h) {
            double sa = 0.0, sd = 0.0;
            for (int64_t bb = 0; bb < b; ++bb) {
                sa += dAbh[bb * H + h];
                sd += dDbh[bb * H + h];
            }
            dA[h] = sa;
            if (dD) dD[h] = sd;
        }
#pragma omp parallel for schedule(static)
        for (int64_t bt = 0; bt < b * L; ++bt)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t n = 0; n < N; ++n) {
                    double sb = 0.0, sc = 0.0;
                    for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
                        sb += dBh[(bt * H + h) * N + n];
                        sc += dCh[(bt * H + h) * N + n];
                    }
                    dB[(bt * G + g) * N + n] = sb;
                    dC[(bt * G + g) * N + n] = sc;
                }
    }
    free(dBh);
    free(dCh);
    free(dAbh);
    free(dDbh);
    return err ? -2 : 0;
}
