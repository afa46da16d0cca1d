// backward.hip -- gradients of the SSD forward (plain input step dt).
//
// Training needs the backward pass, and the forward's intermediate states are
// recomputed rather than stored ("3.3 Hardware-Aware algorithms and GPU memory
// hierarchy optimisation", section 6).  The pass is built on one identity: the
// adjoint of the recurrence S_t = a_t S_{t-1} + dt_t x_t (outer) B_t with
// y_t = C_t . S_t is the same kind of recurrence run backwards in time,
//   G_t = a_{t+1} G_{t+1} + dy_t (outer) C_t,   G_{L-1} includes dfinal,
// so three chunked scans of the forward's own kernels give everything:
//   (b) G in reversed time, read out through B:   u_t = G_t B_t          -> dx
//   (c) G^T in reversed time, read out through x: v_t = G_t^T x_t        -> dB, ddt
//   (d) S^T forwards, read out through dy:        w_t = S_t^T dy_t       -> dC, ddt
// (the transposed scans swap the roles of headdim and dstate, with one B/C
// "group" per head).  The decay gradients follow from the log-decay
// lambda_t = A sum_{k<=t} dt_k, on which the loss depends only through
// differences: d lambda_t = C_t . w_t - dt_t x_t^T G_t B_t (+ <dfinal, S_L-1>
// at the last token), then
//   ddt_k = x_k^T G_k B_k + A sum_{t>=k} d lambda_t,  dA = sum_k dt_k sum_{t>=k} d lambda_t.
// Both flows form the decay gradient chunk by chunk, R_k = a_k <G_k, S_{k-1}>
// expanded over each chunk from its chunk-start state and adjoint (no long suffix
// sum of d lambda, whose terms nearly cancel).  bf16 inputs with headdim 64 and
// dstate 64 or 128 (run_local) use decay_grad.hip and run every scan on the fast
// bf16 chunk kernels, reading the inputs in place (backwards for the reversed
// scans).  Other inputs (run) use the generic chunk kernels in fp32 on
// time-reversed copies of the inputs that this file builds, and a plain fp32
// form of the decay gradient.  The transposed scans' x-role input is B or C of
// the head's group, read through the kernels' x-head map rather than copied per
// head.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace bwd {

// out[b, pad + t, j, k] = in[b, rev ? L-1-t : t, j / rep, k] and zero for the first pad rows (fp32 or bf16
// out, L + pad rows); four consecutive k per thread
template <class T, class O>
__global__ void __launch_bounds__(256) copy_kernel(const T* __restrict__ in, O* __restrict__ out, int64_t b,
                                                   int64_t L, int J, int K, int rep, int rev, int64_t pad,
                                                   int64_t n4) {
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i4 >= n4) return;
    const int64_t e = i4 * 4, Lo = L + pad;
    const int k = (int)(e % K);
    const int j = (int)((e / K) % J);
    const int64_t to = (e / ((int64_t)K * J)) % Lo;
    const int64_t bb = e / ((int64_t)K * J * Lo);
    if (to < pad) {
#pragma unroll
        for (int r = 0; r < 4; ++r) out[e + r] = from_f32<O>(0.0f);
        return;
    }
    const int64_t t = to - pad;
    const int64_t ts = rev ? L - 1 - t : t;
    const int64_t src = ((bb * L + ts) * (J / rep) + j / rep) * K + k;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[e + r] = from_f32<O>(to_f32(in[src + r]));
}

// decay steps of the reversed scans, behind pad rows of zero: d'[b, pad + tau, h] = dt[b, L - tau, h] for
// tau >= 1, 0 at tau = 0 (L + pad rows); and the forward steps as fp32 (L rows)
template <class T>
__global__ void __launch_bounds__(256) steps_kernel(const T* __restrict__ dt, float* __restrict__ drev,
                                                    float* __restrict__ dfwd, int64_t L, int64_t pad, int H,
                                                    int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t Lo = L + pad;
    const int h = (int)(i % H);
    const int64_t to = (i / H) % Lo;
    const int64_t bb = i / ((int64_t)H * Lo);
    const int64_t tau = to - pad;
    drev[i] = tau <= 0 ? 0.0f : to_f32(dt[(bb * L + (L - tau)) * H + h]);
    if (to < L) dfwd[(bb * L + to) * H + h] = to_f32(dt[(bb * L + to) * H + h]);
}

// (b, H, P, N) -> (b, H, N, P), fp32; a NULL source gives zeros
__global__ void __launch_bounds__(256) transpose_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                        int P, int N, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int p = (int)(i % P);
    const int nn = (int)((i / P) % N);
    const int64_t bh = i / ((int64_t)P * N);
    out[i] = in ? in[(bh * P + p) * N + nn] : 0.0f;
}

// the reversed scans' input step is 1 (0 past the sequence end): overwrite dt_t of the chunk cumsum
__global__ void __launch_bounds__(256) ones_kernel(float* __restrict__ dt_t, int64_t L, int Q, int64_t nC, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t pos = i % ((int64_t)nC * Q);  // (c, i) of one (b, h)
    dt_t[i] = pos < L ? 1.0f : 0.0f;
}

// One workgroup per (b, t), all heads: dx = dt u + D dy; per head q = v . B (= x^T G B) and dy . x; per
// group dB = sum_h dt v and dC = sum_h w.  Wavefront wv takes heads
// wv, wv + 4, ... (lanes over p and n) and reads each element of u, v, w once: the group sums
// accumulate in registers while the heads stay in one group (heads are grouped in contiguous
// ranges, so a wavefront meets each group once) and are flushed to a per-wavefront LDS slice.
// Without SLICES (LDS too small for them) the group sums re-read v and w in a second pass.
// u_r and v_r have Lr rows per batch row (time-reversed, behind Lr - L rows of padding).  With u_r NULL
// dx is not written (the adjoint scan wrote it), and with vrev 0 v_r is in forward time (L rows per
// batch row).
template <class T, class U, class V, bool SLICES>
__global__ void __launch_bounds__(256) combine_kernel(const T* __restrict__ dy, const T* __restrict__ x,
                                                      const T* __restrict__ dt, const T* __restrict__ B,
                                                      const float* __restrict__ D,
                                                      const U* __restrict__ u_r, const V* __restrict__ v_r,
                                                      const V* __restrict__ w, T* __restrict__ dx,
                                                      T* __restrict__ dB, T* __restrict__ dC, float* __restrict__ q,
                                                      float* __restrict__ dxy, int64_t L, int64_t Lr, int H, int P,
                                                      int N, int G, int vrev) {
    extern __shared__ float lds[];
    float* sB = lds;                // [G][N]
    float* sdt = sB + G * N;        // [H]
    float* pB = sdt + H;            // [4][G][N] per-wavefront partial dB
    float* pC = pB + 4 * G * N;     // [4][G][N] per-wavefront partial dC
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bt = blockIdx.x;  // b * L + t
    const int64_t bb = bt / L, t = bt % L;
    const int64_t btr = bb * Lr + (Lr - 1 - t), btv = vrev ? btr : bt;
    const int hpg = H / G;
    for (int e = tid; e < G * N; e += 256) sB[e] = to_f32(B[bt * G * N + e]);
    if (SLICES)
        for (int e = tid; e < 8 * G * N; e += 256) pB[e] = 0.0f;  // pB and pC
    for (int h = tid; h < H; h += 256) sdt[h] = to_f32(dt[bt * H + h]);
    __syncthreads();
    constexpr int kMaxNL = 4;  // n = lane + 64 k, N <= 256
    float ab[kMaxNL], ac[kMaxNL];
#pragma unroll
    for (int k = 0; k < kMaxNL; ++k) ab[k] = ac[k] = 0.0f;
    int gcur = wv < H ? wv / hpg : 0;
    auto flush = [&](int g) {
        if (!SLICES) return;
#pragma unroll
        for (int k = 0; k < kMaxNL; ++k) {
            const int n = lane + 64 * k;
            if (n < N) {
                pB[(wv * G + g) * N + n] = ab[k];
                pC[(wv * G + g) * N + n] = ac[k];
            }
            ab[k] = ac[k] = 0.0f;
        }
    };
    for (int h = wv; h < H; h += 4) {
        const int g = h / hpg;
        if (g != gcur) {
            flush(gcur);
            gcur = g;
        }
        const float d = sdt[h], Dh = D ? D[h] : 0.0f;
        float sxy = 0.0f, sq = 0.0f;
        for (int p = lane; p < P; p += 64) {
            const int64_t o = (bt * H + h) * P + p;
            const float gy = to_f32(dy[o]);
            if (u_r) dx[o] = from_f32<T>(fmaf(d, to_f32(u_r[(btr * H + h) * P + p]), Dh * gy));
            sxy = fmaf(gy, to_f32(x[o]), sxy);
        }
#pragma unroll
        for (int k = 0; k < kMaxNL; ++k) {
            const int n = lane + 64 * k;
            if (n < N) {
                const float vv = to_f32(v_r[(btv * H + h) * N + n]), ww = to_f32(w[(bt * H + h) * N + n]);
                sq = fmaf(vv, sB[g * N + n], sq);
                if (SLICES) {
                    ab[k] = fmaf(d, vv, ab[k]);
                    ac[k] += ww;
                }
            }
        }
        // wavefront sums: each 16-lane row by DPP moves, then the four rows
        sq = row16_sum(sq);
        sxy = row16_sum(sxy);
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            sq += __shfl_xor(sq, off, 64);
            sxy += __shfl_xor(sxy, off, 64);
        }
        if (lane == 0) {
            q[(bb * H + h) * L + t] = sq;
            dxy[(bb * H + h) * L + t] = sxy;
        }
    }
    if (wv < H) flush(gcur);
    __syncthreads();
    for (int e = tid; e < G * N; e += 256) {
        float sb = 0.0f, sc = 0.0f;
        if (SLICES) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sb += pB[k * G * N + e];
                sc += pC[k * G * N + e];
            }
        } else {
            const int g = e / N, n = e % N;
            for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
                sb = fmaf(sdt[h], to_f32(v_r[(btv * H + h) * N + n]), sb);
                sc += to_f32(w[(bt * H + h) * N + n]);
            }
        }
        dB[bt * G * N + e] = from_f32<T>(sb);
        dC[bt * G * N + e] = from_f32<T>(sc);
    }
}

// NV consecutive bf16 (8 or 16 bytes) as floats
template <int NV>
__device__ __forceinline__ void ld_bf16(const bf16* p, float* o) {
    if constexpr (NV == 8) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = static_cast<float>(v[i]);
    } else {
        static_assert(NV == 4, "4 or 8 values");
        const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = static_cast<float>(v[i]);
    }
}

// The combine of the chunk-local flow (bf16, dstate N = 64 or 128, H a multiple of 4), one workgroup per
// (b, t), in two halves that run apart: DB, after the adjoint readout v: per head q = v . B and per group
// dB = sum_h dt v; else, after the forward readout w: per group dC = sum_h w.  Four heads at once per
// wavefront, 16 lanes per head: wavefront wv takes the head quads k = wv, wv + 4, ..., lane row r (lane /
// 16) head 4k + r; a lane covers n = (N / 16) l16 .. (16- or 8-byte accesses), so every row of v or w is
// read by one contiguous access per wavefront.  The group sums collect in registers per lane and land, per
// (wavefront, lane row), in an LDS slice when the row's group changes; the slices are added in a fixed
// order at the end.
template <int N, bool DB>
__global__ void __launch_bounds__(256) combine_quad_kernel(const bf16* __restrict__ dt, const bf16* __restrict__ B,
                                                           const bf16* __restrict__ vw, bf16* __restrict__ dBC,
                                                           float* __restrict__ q, int64_t L, int H, int G) {
    constexpr int NV = N / 16;
    extern __shared__ float lds[];
    float* pS = lds;  // [16][G][N] per-(wavefront, lane row) partial dB or dC
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane >> 4, l16 = lane & 15;
    const int slot = 4 * wv + r;
    const int64_t bt = blockIdx.x;  // b * L + t
    const int64_t bb = bt / L, t = bt % L;
    const int hpg = H / G, nq = H / 4;
    // with one group and every (wavefront, lane row) slot holding heads, every slot writes its partial sums
    if (!(G == 1 && nq >= 4)) {
        for (int e = tid; e < 16 * G * N; e += 256) lds[e] = 0.0f;
        __syncthreads();
    }
    float acc[NV], bv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.0f;
    int gcur = -1;
    for (int qd = wv; qd < nq; qd += 4) {
        const int h = 4 * qd + r, g = h / hpg;
        if (g != gcur) {  // the same in each lane row
            if (gcur >= 0) {
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    pS[(slot * G + gcur) * N + NV * l16 + k] = acc[k];
                    acc[k] = 0.0f;
                }
            }
            gcur = g;
            if constexpr (DB) ld_bf16<NV>(B + (bt * G + g) * N + NV * l16, bv);
        }
        float vv[NV];
        ld_bf16<NV>(vw + (bt * H + h) * N + NV * l16, vv);
        if constexpr (DB) {
            const float d = static_cast<float>(dt[bt * H + h]);
            float sq = 0.0f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                sq = fmaf(vv[k], bv[k], sq);
                acc[k] = fmaf(d, vv[k], acc[k]);
            }
            sq = row16_sum(sq);
            if (l16 == 0) q[(bb * H + h) * L + t] = sq;
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] += vv[k];
        }
    }
    if (gcur >= 0) {
#pragma unroll
        for (int k = 0; k < NV; ++k) pS[(slot * G + gcur) * N + NV * l16 + k] = acc[k];
    }
    __syncthreads();
    for (int e = tid; e < G * N; e += 256) {
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) sum += pS[k * G * N + e];
        dBC[bt * G * N + e] = static_cast<bf16>(sum);
    }
}

// the combine kernel with LDS slices for the group sums when they fit, else the two-pass form
template <class T, class U, class V>
hipError_t launch_combine(const void* dy, const void* x, const void* dt, const void* B, const float* D, const U* u_r,
                          const V* v_r, const V* w, void* dx, void* dB, void* dC, float* q, float* dxy, int64_t b,
                          int64_t L, int64_t Lr, int H, int P, int N, int G, hipStream_t st, bool vrev = true) {
    const size_t base = (size_t)(G * N + H) * 4, sliced = base + (size_t)8 * G * N * 4;
    const bool slices = sliced <= 160 * 1024;
    const size_t lds = slices ? sliced : base;
    const void* fn =
        slices ? (const void*)combine_kernel<T, U, V, true> : (const void*)combine_kernel<T, U, V, false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (slices)
        hipLaunchKernelGGL((combine_kernel<T, U, V, true>), dim3((unsigned)(b * L)), dim3(256), lds, st,
                           static_cast<const T*>(dy), static_cast<const T*>(x), static_cast<const T*>(dt),
                           static_cast<const T*>(B), D, u_r, v_r, w, static_cast<T*>(dx), static_cast<T*>(dB),
                           static_cast<T*>(dC), q, dxy, L, Lr, H, P, N, G, vrev ? 1 : 0);
    else
        hipLaunchKernelGGL((combine_kernel<T, U, V, false>), dim3((unsigned)(b * L)), dim3(256), lds, st,
                           static_cast<const T*>(dy), static_cast<const T*>(x), static_cast<const T*>(dt),
                           static_cast<const T*>(B), D, u_r, v_r, w, static_cast<T*>(dx), static_cast<T*>(dB),
                           static_cast<T*>(dC), q, dxy, L, Lr, H, P, N, G, vrev ? 1 : 0);
    return hipGetLastError();
}

// The chunk-local decay gradient for the fp32 flow (any headdim, dstate and chunk up to 512), the same four
// terms as decay_grad.hip, R_k = T1 + T2_k + T3_k + T4_k, in plain fp32 loops; one workgroup per (head,
// chunk, b).  The in-chunk cumulative log2 decay is formed here in fp64 from dt, so the decay between any
// two tokens of the chunk is exact to fp32 rounding however large the chunk's total.  S0T: the forward
// transposed scan's chunk-start states (b, nC, H, N, P); Gst: the adjoint scan's chunk-start states
// (b, nC, H, P, N) in reversed chunk order (its walk front-padded to whole chunks), entering decayed by
// the next chunk's first token; the last chunk's is dfinal.
template <class T>
__global__ void __launch_bounds__(256) decay_grad_plain_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                                                               const T* __restrict__ B, const T* __restrict__ C,
                                                               const T* __restrict__ dt, const float* __restrict__ A,
                                                               const float* __restrict__ S0T,
                                                               const float* __restrict__ Gst, float* __restrict__ R,
                                                               int64_t L, int H, int P, int N, int G, int Q,
                                                               int64_t nC) {
    extern __shared__ double dsm[];
    double* lw = dsm;          // [Q] in-chunk cumulative log2 decay, fp64 (flat past the sequence end)
    double* t2 = lw + Q;       // [Q] T2 suffix sums
    double* red = t2 + Q;      // [256]
    float* dtw = reinterpret_cast<float*>(red + 256);  // [Q]
    float *s2 = dtw + Q, *s3 = s2 + Q, *rowsum = s3 + Q, *colsum = rowsum + Q;
    const int tid = threadIdx.x, h = blockIdx.x;
    const int64_t c = blockIdx.y, bb = blockIdx.z;
    const int g = h / (H / G);
    const int64_t c0 = c * Q;
    const int valid = (int)(L - c0 < Q ? L - c0 : Q);
    const double al = (double)A[h] * 1.4426950408889634;  // A log2 e
    for (int t = tid; t < Q; t += 256) {
        dtw[t] = t < valid ? to_f32(dt[(bb * L + c0 + t) * H + h]) : 0.0f;
        s2[t] = s3[t] = rowsum[t] = colsum[t] = 0.0f;
    }
    __syncthreads();
    if (tid == 0) {
        double acc = 0.0;
        for (int t = 0; t < Q; ++t) {
            acc += al * (double)dtw[t];
            lw[t] = acc;
        }
    }
    // T1's dot <Gam, S0> in fp64
    const int64_t PN = (int64_t)P * N, HP = (int64_t)H * P, GN = (int64_t)G * N;
    const float* S0c = S0T + ((bb * nC + c) * H + h) * PN;           // [n][p]
    const float* Gc = Gst + ((bb * nC + (nC - 1 - c)) * H + h) * PN;  // [p][n]
    double dot = 0.0;
    for (int64_t e = tid; e < PN; e += 256) dot += (double)Gc[e] * (double)S0c[(e % N) * P + e / N];
    red[tid] = dot;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    const double tdot = red[0];
    // s2_t = dy_t . (S0 C_t) and s3_t = x_t . (Gam B_t), one (token, p) per step
    for (int e = tid; e < valid * P; e += 256) {
        const int t = e / P, p = e % P;
        const T* Ct = C + (bb * L + c0 + t) * GN + (int64_t)g * N;
        const T* Bt = B + (bb * L + c0 + t) * GN + (int64_t)g * N;
        float u = 0.0f, v = 0.0f;
        for (int n = 0; n < N; ++n) {
            u = fmaf(S0c[(int64_t)n * P + p], to_f32(Ct[n]), u);
            v = fmaf(Gc[(int64_t)p * N + n], to_f32(Bt[n]), v);
        }
        const int64_t o = (bb * L + c0 + t) * HP + (int64_t)h * P + p;
        atomicAdd(&s2[t], to_f32(dy[o]) * u);
        atomicAdd(&s3[t], to_f32(x[o]) * v);
    }
    // T4: M_tj = (dy_t . x_j)(C_t . B_j) 2^(l_t - l_j) dt_j over the pairs j < t, into row and column sums
    const int npair = valid * (valid - 1) / 2;
    for (int e = tid; e < npair; e += 256) {
        int t = (int)((1.0 + sqrt(1.0 + 8.0 * (double)e)) * 0.5);  // pair e = t (t - 1) / 2 + j
        while (t * (t - 1) / 2 > e) --t;
        while ((t + 1) * t / 2 <= e) ++t;
        const int j = e - t * (t - 1) / 2;
        const T* yt = dy + (bb * L + c0 + t) * HP + (int64_t)h * P;
        const T* xj = x + (bb * L + c0 + j) * HP + (int64_t)h * P;
        const T* Ct = C + (bb * L + c0 + t) * GN + (int64_t)g * N;
        const T* Bj = B + (bb * L + c0 + j) * GN + (int64_t)g * N;
        float yx = 0.0f, cb = 0.0f;
        for (int p = 0; p < P; ++p) yx = fmaf(to_f32(yt[p]), to_f32(xj[p]), yx);
        for (int n = 0; n < N; ++n) cb = fmaf(to_f32(Ct[n]), to_f32(Bj[n]), cb);
        const float m = yx * cb * exp2f((float)(lw[t] - lw[j])) * dtw[j];
        atomicAdd(&rowsum[t], m);
        atomicAdd(&colsum[j], m);
    }
    __syncthreads();
    // R_k = T1 + T2_k + T3_k + T4_k, in fp64 over the chunk's positions
    if (tid == 0) {
        const double lend = lw[Q - 1];
        // the adjoint enters decayed by the next token's factor (none after the sequence's end)
        const double gam = c + 1 < nC ? exp2(al * (double)to_f32(dt[(bb * L + c0 + Q) * H + h])) : 1.0;
        const double T1 = exp2(lend) * gam * tdot;
        double suf = 0.0;
        for (int k = valid - 1; k >= 0; --k) {
            suf += exp2(lw[k]) * (double)s2[k];
            t2[k] = suf;
        }
        double pre3 = 0.0, pre4 = 0.0;
        float* Rh = R + (bb * H + h) * L + c0;
        for (int k = 0; k < valid; ++k) {
            Rh[k] = (float)(T1 + t2[k] + pre3 + pre4);
            pre3 += (double)dtw[k] * exp2(lend - lw[k]) * gam * (double)s3[k];
            pre4 += (double)colsum[k] - (double)rowsum[k];
        }
    }
}

inline size_t decay_grad_plain_lds(int Q) { return (size_t)(2 * Q + 256) * 8 + (size_t)5 * Q * 4; }

// dA[h], dD[h]: sums over the batch rows
__global__ void __launch_bounds__(256) reduce_kernel(const double* __restrict__ dA_part, const double* __restrict__ dD_part,
                                                     float* __restrict__ dA, float* __restrict__ dD, int64_t b, int H) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    double sa = 0.0, sd = 0.0;
    for (int64_t bb = 0; bb < b; ++bb) {
        sa += dA_part[bb * H + h];
        sd += dD_part[bb * H + h];
    }
    dA[h] = (float)sa;
    if (dD) dD[h] = (float)sd;
}

// dh0 = a_0 G_0 (G_0: the reversed adjoint scan's final state); with no tokens, dh0 = dfinal
// The chunk-local decay gradient's last step, one workgroup per (b, h): ddt = q + A R per token, and the
// partial sums dA = sum dt R, dD = sum dy . x (fp64).
template <class T>
__global__ void __launch_bounds__(256) finish_kernel(const float* __restrict__ q, const float* __restrict__ R,
                                                     const float* __restrict__ dxy, const T* __restrict__ dt,
                                                     const float* __restrict__ A, T* __restrict__ ddt,
                                                     double* __restrict__ dA_part, double* __restrict__ dD_part,
                                                     int64_t L, int H) {
    __shared__ double red[2][256];
    const int tid = threadIdx.x, h = blockIdx.x;
    const int64_t bb = blockIdx.y, bh = bb * H + h;
    const double Ah = A[h];
    double da = 0.0, dd = 0.0;
    for (int64_t t = tid; t < L; t += 256) {
        const double r = R[bh * L + t];
        ddt[(bb * L + t) * H + h] = from_f32<T>((float)(Ah * r + (double)q[bh * L + t]));
        da += (double)to_f32(dt[(bb * L + t) * H + h]) * r;
        dd += (double)dxy[bh * L + t];
    }
    red[0][tid] = da;
    red[1][tid] = dd;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) {
            red[0][tid] += red[0][tid + s];
            red[1][tid] += red[1][tid + s];
        }
        __syncthreads();
    }
    if (tid == 0) {
        dA_part[bh] = red[0][0];
        dD_part[bh] = red[1][0];
    }
}

// The same over a tile of kFinTok tokens and every head, one workgroup per (b, tile), with per-tile
// partial sums: q, R and dxy ((b, H, L)) are read along the tokens and dt, ddt ((b, L, H)) along the heads,
// both coalesced, through an LDS tile [4][H][kFinTok + 1].
constexpr int kFinTok = 32;

template <class T>
__global__ void __launch_bounds__(256) finish_tile_kernel(const float* __restrict__ q, const float* __restrict__ R,
                                                          const float* __restrict__ dxy, const T* __restrict__ dt,
                                                          const float* __restrict__ A, T* __restrict__ ddt,
                                                          double* __restrict__ dA_part, double* __restrict__ dD_part,
                                                          int64_t L, int H, int64_t ntile) {
    constexpr int TS = kFinTok + 1;
    extern __shared__ float lds[];
    float *Rl = lds, *ql = Rl + H * TS, *xl = ql + H * TS, *dl = xl + H * TS;
    const int tid = threadIdx.x;
    const int64_t tile = blockIdx.x, bb = blockIdx.y, t0 = tile * kFinTok;
    for (int e = tid; e < H * kFinTok; e += 256) {
        const int h = e / kFinTok, tt = e % kFinTok;
        const int64_t t = t0 + tt, o = (bb * H + h) * L + t;
        const bool in = t < L;
        Rl[h * TS + tt] = in ? R[o] : 0.0f;
        ql[h * TS + tt] = in ? q[o] : 0.0f;
        xl[h * TS + tt] = in ? dxy[o] : 0.0f;
    }
    __syncthreads();
    for (int e = tid; e < H * kFinTok; e += 256) {
        const int tt = e / H, h = e % H;
        const int64_t t = t0 + tt;
        float d = 0.0f;
        if (t < L) {
            const int64_t o = (bb * L + t) * H + h;
            const float r = Rl[h * TS + tt];
            ddt[o] = from_f32<T>((float)((double)A[h] * r + (double)ql[h * TS + tt]));
            d = to_f32(dt[o]);
        }
        dl[h * TS + tt] = d;
    }
    __syncthreads();
    for (int h = tid; h < H; h += 256) {
        double da = 0.0, dd = 0.0;
        for (int tt = 0; tt < kFinTok; ++tt) {
            da += (double)dl[h * TS + tt] * (double)Rl[h * TS + tt];
            dd += (double)xl[h * TS + tt];
        }
        dA_part[(bb * ntile + tile) * H + h] = da;
        dD_part[(bb * ntile + tile) * H + h] = dd;
    }
}

// dA[h], dD[h]: sums of the rows partial sums, one workgroup per head (fp64)
__global__ void __launch_bounds__(256) reduce_rows_kernel(const double* __restrict__ dA_part,
                                                          const double* __restrict__ dD_part, float* __restrict__ dA,
                                                          float* __restrict__ dD, int64_t rows, int H) {
    __shared__ double red[2][256];
    const int tid = threadIdx.x, h = blockIdx.x;
    double sa = 0.0, sd = 0.0;
    for (int64_t r = tid; r < rows; r += 256) {
        sa += dA_part[r * H + h];
        sd += dD_part[r * H + h];
    }
    red[0][tid] = sa;
    red[1][tid] = sd;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) {
            red[0][tid] += red[0][tid + s];
            red[1][tid] += red[1][tid + s];
        }
        __syncthreads();
    }
    if (tid == 0) {
        dA[h] = (float)red[0][0];
        if (dD) dD[h] = (float)red[1][0];
    }
}

inline size_t finish_tile_lds(int H) { return (size_t)4 * H * (kFinTok + 1) * 4; }

template <class T>
__global__ void __launch_bounds__(256) dh0_kernel(const float* __restrict__ G0, const T* __restrict__ dt,
                                                  const float* __restrict__ A, const float* __restrict__ dfinal,
                                                  float* __restrict__ dh0, int64_t L, int H, int64_t PN, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t bh = i / PN;
    const int h = (int)(bh % H);
    const int64_t bb = bh / H;
    if (L == 0) {
        dh0[i] = dfinal ? dfinal[i] : 0.0f;
        return;
    }
    dh0[i] = fast_exp2(to_f32(dt[(bb * L) * H + h]) * A[h] * kLog2e) * G0[i];
}

inline dim3 grid1(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

template <class T, class O = float>
hipError_t copy(const void* in, O* out, int64_t b, int64_t L, int J, int K, int rep, bool rev, int64_t pad,
                hipStream_t st) {
    const int64_t n4 = b * (L + pad) * J * (int64_t)K / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL((copy_kernel<T, O>), grid1(n4), dim3(256), 0, st, static_cast<const T*>(in), out, b, L, J, K, rep,
                       rev ? 1 : 0, pad, n4);
    return hipGetLastError();
}

// one chunked scan (cumsum arrays given): chunk states, state pass from h0, chunk output
hipError_t scan(const Shape& s, const void* xin, const void* Bin, const void* Cin, const float* dt_t,
                const float* cs, float* states, const float* h0, float* fin, void* y, hipStream_t st) {
    hipError_t e = launch_chunk_state(s, xin, Bin, dt_t, cs, states, st);
    if (e != hipSuccess) return e;
    e = launch_state_passing(s, states, cs, h0, fin, st);
    if (e != hipSuccess) return e;
    return launch_chunk_scan(s, xin, Bin, Cin, dt_t, cs, states, nullptr, y, st);
}

// the same on the generic kernels with fp32 compute, inputs of dtype in_io, x-head map xrep
hipError_t scan_in(const Shape& s, int in_io, int xrep, const void* xin, const void* Bin, const void* Cin,
                   const float* dt_t, const float* cs, float* states, const float* h0, float* fin, void* y,
                   hipStream_t st) {
    hipError_t e = launch_chunk_state_in(s, in_io, xrep, xin, Bin, dt_t, cs, states, st);
    if (e != hipSuccess) return e;
    e = launch_state_passing(s, states, cs, h0, fin, st);
    if (e != hipSuccess) return e;
    return launch_chunk_scan_in(s, in_io, xrep, xin, Bin, Cin, dt_t, cs, states, nullptr, y, st);
}

// dh0 = a_0 G_0 from the transposed adjoint of a transposed scan's final state G0T (b, (N / 64) H, 64, P):
// element (p, n) of head h sits at half-head h (N / 64) + n / 64, row n % 64; with no tokens dh0 = dfinal
template <class T>
__global__ void __launch_bounds__(256) dh0_tr_kernel(const float* __restrict__ G0T, const T* __restrict__ dt,
                                                     const float* __restrict__ A, const float* __restrict__ dfinal,
                                                     float* __restrict__ dh0, int64_t L, int H, int P, int N,
                                                     int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int nn = (int)(i % N);
    const int p = (int)((i / N) % P);
    const int64_t bh = i / ((int64_t)P * N);
    const int h = (int)(bh % H);
    const int64_t bb = bh / H;
    if (L == 0) {
        dh0[i] = dfinal ? dfinal[i] : 0.0f;
        return;
    }
    const float g = G0T[((bh * (N / 64) + nn / 64) * 64 + nn % 64) * P + p];
    dh0[i] = fast_exp2(to_f32(dt[(bb * L) * H + h]) * A[h] * kLog2e) * g;
}

// The backward with the decay gradient formed chunk by chunk (decay_grad.hip), for bf16 io with headdim
// 64 and dstate 64 or 128.  The decay gradient then needs no long suffix sum, so the transposed scans
// (c) and (d), which only feed dB, dC and q, run in bf16 compute.  Every scan reads the inputs in place
// and uses sub-chunk-local decay arrays (exact in-chunk decays at any chunk length).  The reversed scans
// walk the inputs backwards (XMap::rows) over Lr tokens, the sequence front-padded to whole backward
// chunks of Q tokens (the padding reads as zero), so that every reversed Q-chunk is a forward Q-chunk read
// backwards.  The decay gradient needs, at every Q-chunk, the forward state entering it (S0) and the
// adjoint entering it from the next one: both are stored every Q tokens by scans that carry that state in
// registers at the transposed scans' large chunk (hi/lo state updates) -- the adjoint scan (b), and the
// forward transposed scan (d), whose state is S^T and is stored back in (P, N) layout -- so there are
// no Q-chunk local states and no pass over them.
}  // namespace bwd

// The local flow's combine in two halves (dC after the forward readout, dB and q after the adjoint one):
// headdim 64, dstate 64 or 128, H a multiple of 4, and one LDS slice set per (wavefront, lane row) and
// group within 64 KB.
static size_t quad_combine_lds(const Shape& s) { return (size_t)16 * s.G * s.N * 4; }
static bool quad_combine(const Shape& s) {
    return s.P == 64 && (s.N == 64 || s.N == 128) && s.H % 4 == 0 && quad_combine_lds(s) <= 64 * 1024;
}

namespace bwd {

hipError_t run_local(const Shape& s, const BackwardLayout& f, const void* x, const void* dt, const float* A,
                     const void* B, const void* C, const float* D, const float* h0, const void* dy,
                     const float* dfinal, void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0,
                     char* ws, hipStream_t st) {
    using T = bf16;
    const int64_t b = s.b, L = s.L, Lr = f.Lr;
    const int H = (int)s.H, P = (int)s.P, N = (int)s.N, G = (int)s.G;
    const int nh = N / 64, H2 = nh * H, hpg = H / G;
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    float *states = F(f.states), *states_b = F(f.states_b), *R = F(f.R);
    float *G0T = F(f.G0), *dfT = F(f.dfT), *h0T = F(f.h0T), *finT = F(f.finT), *q = F(f.q), *dxy = F(f.dxy);
    float *totals = F(f.totals), *stT = F(f.stT);
    T *v = reinterpret_cast<T*>(ws + f.v_r), *w = reinterpret_cast<T*>(ws + f.w);
    double *dA_part = reinterpret_cast<double*>(ws + f.dA_part), *dD_part = reinterpret_cast<double*>(ws + f.dD_part);
    // the sub-chunk-local decay arrays (dtl, lw pairs): reversed per head (b), reversed per half-head (c),
    // forwards per half-head (d); the per-head and per-half-head ones coincide at N = 64
    // (a pair for k heads over n sub-chunks: dtl, then lw, each b k n 64 floats; backward_layout sizes them)
    const int64_t nsr = Lr / 64, nsf = (L + 63) / 64;
    float* at = F(f.sub);
    auto pair = [&](int64_t heads, int64_t nsub) {
        float* p = at;
        at += 2 * b * heads * nsub * 64;
        return p;
    };
    float* rl = pair(H, nsr);
    float* rh = nh == 2 ? pair(H2, nsr) : rl;
    float* fh = pair(H2, nsf);
    auto dtl = [](float* p) { return p; };
    auto lwp = [](float* p, int64_t heads, int64_t nsub, int64_t bb) { return p + bb * heads * nsub * 64; };
    const int64_t PN = (int64_t)P * N;
    hipError_t e;
#define BWD_CHECK(expr)                \
    do {                               \
        e = (expr);                    \
        if (e != hipSuccess) return e; \
    } while (0)
    hipLaunchKernelGGL(transpose_kernel, grid1(b * H * PN), dim3(256), 0, st, dfinal, dfT, P, N, b * H * PN);
    BWD_CHECK(hipGetLastError());
    hipLaunchKernelGGL(transpose_kernel, grid1(b * H * PN), dim3(256), 0, st, h0, h0T, P, N, b * H * PN);
    BWD_CHECK(hipGetLastError());

    // the decay arrays in one launch: reversed per head (b), reversed per half-head (c), forwards per
    // half-head (d) (at N = 64 the half-heads are the heads and the second set is the first)
    DecaySet sets[3];
    int nsets = 0;
    sets[nsets++] = DecaySet{dtl(rl), lwp(rl, H, nsr, b), b, Lr, L, H, 1, true, true};
    if (nh == 2) sets[nsets++] = DecaySet{dtl(rh), lwp(rh, H2, nsr, b), b, Lr, L, H2, 2, true, true};
    sets[nsets++] = DecaySet{dtl(fh), lwp(fh, H2, nsf, b), b, L, L, H2, nh, false, false};
    BWD_CHECK(launch_subchunk_decay_bwd_sets(sets, nsets, dt, A, st));

    // The half-head scans (c) and (d): H2 half-heads of headdim 64 (at dstate 128 each head splits into the
    // two halves of the state's N rows, which form one head pair) whose x is (that half of) B or C of the
    // head's group.
    Shape sh = s;
    sh.H = H2;
    sh.P = 64;
    sh.N = P;
    sh.G = H;
    Shape s1;  // the pass over the chunk totals: a chunk of "length 1" in its indexing
    const bool split = quad_combine(s);
    const bf16 *dtb = static_cast<const bf16*>(dt), *Bb = static_cast<const bf16*>(B);
    const unsigned nbt = (unsigned)(b * L);
    const size_t lq = quad_combine_lds(s);
    // (d) S^T read out through dy: w (dC), forwards in time; it also stores the forward state entering every
    // Q-chunk (S0), back in the heads' (P, N) layout.  With the split combine, dC is summed at once and w's
    // memory then serves v and the adjoint's states.
    sh.L = L;
    sh.Q = f.Qt;
    sh.nC = (L + f.Qt - 1) / f.Qt;
    s1 = sh;
    s1.Q = 1;
    const XMap xm{nh * G, nh * hpg, nh, 0, nullptr, nullptr, 0, 0, 0};
    const XMap xmt{nh * G, nh * hpg, nh, 0, nullptr, states, (int)s.Q, 0, nh};
    BWD_CHECK(launch_chunk_state_sub(sh, B, x, dtl(fh), lwp(fh, H2, nsf, b), stT, totals, st, &xm));
    BWD_CHECK(launch_state_passing(s1, stT, totals, h0 ? h0T : nullptr, finT, st));
    BWD_CHECK(launch_chunk_scan_sub(sh, B, x, dy, dtl(fh), lwp(fh, H2, nsf, b), stT, nullptr, w, st, &xmt));
    if (split) {
        if (N == 128)
            hipLaunchKernelGGL((combine_quad_kernel<128, false>), dim3(nbt), dim3(256), lq, st, dtb, Bb, w,
                               static_cast<bf16*>(dC), q, L, H, G);
        else
            hipLaunchKernelGGL((combine_quad_kernel<64, false>), dim3(nbt), dim3(256), lq, st, dtb, Bb, w,
                               static_cast<bf16*>(dC), q, L, H, G);
        BWD_CHECK(hipGetLastError());
    }
    // (c) G^T read out through x: v (dB, q), reversed, written forwards.  Its chunk-start states seed the
    // adjoint scan (b) and its final state is the adjoint at the first token (dh0).
    sh.L = Lr;
    sh.nC = (Lr + f.Qt - 1) / f.Qt;
    s1 = sh;
    s1.Q = 1;
    const XMap xmr{nh * G, nh * hpg, nh, L, nullptr, nullptr, 0, 0, 0};
    BWD_CHECK(launch_chunk_state_sub(sh, C, dy, dtl(rh), lwp(rh, H2, nsr, b), stT, totals, st, &xmr));
    BWD_CHECK(launch_state_passing(s1, stT, totals, dfT, G0T, st));
    BWD_CHECK(launch_chunk_scan_sub(sh, C, dy, x, dtl(rh), lwp(rh, H2, nsr, b), stT, nullptr, v, st, &xmr));
    if (split) {
        if (N == 128)
            hipLaunchKernelGGL((combine_quad_kernel<128, true>), dim3(nbt), dim3(256), lq, st, dtb, Bb, v,
                               static_cast<bf16*>(dB), q, L, H, G);
        else
            hipLaunchKernelGGL((combine_quad_kernel<64, true>), dim3(nbt), dim3(256), lq, st, dtb, Bb, v,
                               static_cast<bf16*>(dB), q, L, H, G);
        BWD_CHECK(hipGetLastError());
    }
    // (b) the adjoint G read out through B: dx = dt u + D dy written by the scan itself (u = G B, dt as the
    // output row scale, D on the x-role dy), started from (c)'s states and storing the adjoint entering
    // every Q-chunk in states_b
    Shape sb = s;
    sb.L = Lr;
    sb.Q = f.Qt;
    sb.nC = sh.nC;
    const XMap xb{H, 1, 1, L, dt, states_b, (int)s.Q, 1, 0};
    BWD_CHECK(launch_chunk_scan_sub(sb, dy, C, B, dtl(rl), lwp(rl, H, nsr, b), stT, D, dx, st, &xb));
    // the decay gradient, chunk by chunk at Q, from the steps and the stored states
    BWD_CHECK(launch_decay_grad(s, x, dy, B, C, dt, A, states, states_b, F(f.cbt), R, dxy, st));
    if (!split)
        BWD_CHECK((launch_combine<T, bf16, bf16>(dy, x, dt, B, D, nullptr, v, w, dx, dB, dC, q, dxy, b, L, L, H, P, N,
                                                 G, st, false)));
    if (finish_tile_lds(H) <= 64 * 1024) {
        const int64_t ntile = (L + kFinTok - 1) / kFinTok;
        hipLaunchKernelGGL(finish_tile_kernel<T>, dim3((unsigned)ntile, (unsigned)b), dim3(256), finish_tile_lds(H),
                           st, q, R, dxy, static_cast<const T*>(dt), A, static_cast<T*>(ddt), dA_part, dD_part, L, H,
                           ntile);
        BWD_CHECK(hipGetLastError());
        hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)H), dim3(256), 0, st, dA_part, dD_part, dA, dD,
                           b * ntile, H);
    } else {
        hipLaunchKernelGGL(finish_kernel<T>, dim3((unsigned)H, (unsigned)b), dim3(256), 0, st, q, R, dxy,
                           static_cast<const T*>(dt), A, static_cast<T*>(ddt), dA_part, dD_part, L, H);
        BWD_CHECK(hipGetLastError());
        hipLaunchKernelGGL(reduce_kernel, grid1(H), dim3(256), 0, st, dA_part, dD_part, dA, dD, b, H);
    }
    BWD_CHECK(hipGetLastError());
    if (dh0) {
        hipLaunchKernelGGL(dh0_tr_kernel<T>, grid1(b * H * PN), dim3(256), 0, st, G0T, static_cast<const T*>(dt), A,
                           dfinal, dh0, L, H, P, N, b * H * PN);
        BWD_CHECK(hipGetLastError());
    }
    (void)H2;
#undef BWD_CHECK
    return hipSuccess;
}

template <class T>
hipError_t run(const Shape& s, const BackwardLayout& f, const void* x, const void* dt, const float* A,
               const void* B, const void* C, const float* D, const float* h0, const void* dy, const float* dfinal,
               void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, char* ws, hipStream_t st) {
    const int64_t b = s.b, L = s.L, Lr = f.Lr, pad = f.Lr - s.L;
    const int H = (int)s.H, P = (int)s.P, N = (int)s.N, G = (int)s.G;
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    T *xr = reinterpret_cast<T*>(ws + f.xr), *dyr = reinterpret_cast<T*>(ws + f.dyr);
    T *Cr = reinterpret_cast<T*>(ws + f.Cr), *Br = reinterpret_cast<T*>(ws + f.Br);
    float *drev = F(f.drev), *dfwd = F(f.dfwd), *dt_t = F(f.dt_t), *cs = F(f.cs);
    float *states = F(f.states), *states_b = F(f.states_b), *u_r = F(f.u_r), *v_r = F(f.v_r), *w = F(f.w);
    float *G0 = F(f.G0), *dfT = F(f.dfT), *h0T = F(f.h0T), *finT = F(f.finT), *fscr = F(f.fscr), *q = F(f.q);
    float *dxy = F(f.dxy), *R = F(f.R);
    double *dA_part = reinterpret_cast<double*>(ws + f.dA_part), *dD_part = reinterpret_cast<double*>(ws + f.dD_part);
    const int64_t PN = (int64_t)P * N;
    const int io = sizeof(T) == 2 ? 1 : 0;
    hipError_t e;
#define BWD_CHECK(expr)             \
    do {                            \
        e = (expr);                 \
        if (e != hipSuccess) return e; \
    } while (0)
    if (L == 0 || b == 0) {
        // no tokens or no rows: zero gradients of the parameters (a sum over nothing), dh0 = dfinal
        hipLaunchKernelGGL(reduce_kernel, grid1(H), dim3(256), 0, st, (const double*)nullptr, (const double*)nullptr,
                           dA, dD, (int64_t)0, H);
        BWD_CHECK(hipGetLastError());
        if (dh0 && b > 0) {
            hipLaunchKernelGGL(dh0_kernel<T>, grid1(b * H * PN), dim3(256), 0, st, (const float*)nullptr,
                               static_cast<const T*>(dt), A, dfinal, dh0, (int64_t)0, H, PN, b * H * PN);
            BWD_CHECK(hipGetLastError());
        }
        return hipSuccess;
    }
    // time-reversed copies for the reversed scans, in the input dtype, front-padded to whole chunks so that
    // every reversed chunk is a forward chunk read backwards
    BWD_CHECK((copy<T, T>(x, xr, b, L, H, P, 1, true, pad, st)));
    BWD_CHECK((copy<T, T>(dy, dyr, b, L, H, P, 1, true, pad, st)));
    BWD_CHECK((copy<T, T>(C, Cr, b, L, G, N, 1, true, pad, st)));
    BWD_CHECK((copy<T, T>(B, Br, b, L, G, N, 1, true, pad, st)));
    hipLaunchKernelGGL(steps_kernel<T>, grid1(b * Lr * H), dim3(256), 0, st, static_cast<const T*>(dt), drev, dfwd, L,
                       pad, H, b * Lr * H);
    BWD_CHECK(hipGetLastError());
    hipLaunchKernelGGL(transpose_kernel, grid1(b * H * PN), dim3(256), 0, st, dfinal, dfT, P, N, b * H * PN);
    BWD_CHECK(hipGetLastError());
    hipLaunchKernelGGL(transpose_kernel, grid1(b * H * PN), dim3(256), 0, st, h0, h0T, P, N, b * H * PN);
    BWD_CHECK(hipGetLastError());

    const DtFront none{nullptr, 0, 0, 0, 0.0f, 0.0f};
    Shape sb = s;  // the adjoint scan: headdim P, dstate N, G groups, fp32 compute, over Lr reversed tokens
    sb.io = 0;
    sb.L = Lr;
    Shape sT = sb;  // the transposed scans: headdim N, dstate P, one group per head
    sT.P = N;
    sT.N = P;
    sT.G = H;
    const int hpg = H / G;  // the transposed scans' x-role (B or C) is shared by the heads of a group
    // reversed scans (b) and (c): decay steps d', input step 1
    BWD_CHECK(launch_chunk_cumsum(sb, none, drev, A, dt_t, cs, st));
    hipLaunchKernelGGL(ones_kernel, grid1(b * H * s.nC * s.Q), dim3(256), 0, st, dt_t, Lr, (int)s.Q, s.nC,
                       b * H * s.nC * s.Q);
    BWD_CHECK(hipGetLastError());
    // (b) on the bf16 chunk kernels when the shape allows: dx (bf16 accuracy), and the final adjoint and the
    // chunk-start adjoints (fp32, hi + lo split chunk states) for the decay gradient
    Shape s16 = sb;
    s16.io = 1;
    const bool fastb = io == 1 && fast_chunk_supported(s16);
    if (fastb)
        BWD_CHECK(scan(s16, dyr, Cr, Br, dt_t, cs, states_b, dfinal, G0, u_r, st));
    else
        BWD_CHECK(scan_in(sb, io, 1, dyr, Cr, Br, dt_t, cs, states_b, dfinal, G0, u_r, st));
    // (c): x-role C of the head's group, B-role dy, read out through x (all reversed)
    BWD_CHECK(scan_in(sT, io, hpg, Cr, dyr, xr, dt_t, cs, states, dfT, fscr, v_r, st));
    // forward transposed scan (d): decay and input step dt; x-role B, B-role x, read out through dy; its
    // chunk-start states (S0 transposed) stay in `states` for the decay gradient
    Shape sf = s;
    sf.io = 0;
    Shape sTf = sT;
    sTf.L = L;
    BWD_CHECK(launch_chunk_cumsum(sf, none, dfwd, A, dt_t, cs, st));
    BWD_CHECK(scan_in(sTf, io, hpg, B, x, dy, dt_t, cs, states, h0 ? h0T : nullptr, finT, w, st));

    // combine: dx, dB, dC, q and dy . x
    if (fastb)
        BWD_CHECK((launch_combine<T, bf16, float>(dy, x, dt, B, D, reinterpret_cast<const bf16*>(u_r), v_r, w, dx, dB,
                                                  dC, q, dxy, b, L, Lr, H, P, N, G, st)));
    else
        BWD_CHECK((launch_combine<T, float, float>(dy, x, dt, B, D, u_r, v_r, w, dx, dB, dC, q, dxy, b, L, Lr, H, P,
                                                   N, G, st)));
    // the decay gradient chunk by chunk, then ddt, dA, dD
    const size_t lds = decay_grad_plain_lds((int)s.Q);
    BWD_CHECK(hipFuncSetAttribute((const void*)decay_grad_plain_kernel<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds));
    hipLaunchKernelGGL(decay_grad_plain_kernel<T>, dim3((unsigned)H, (unsigned)s.nC, (unsigned)b), dim3(256), lds, st,
                       static_cast<const T*>(x), static_cast<const T*>(dy), static_cast<const T*>(B),
                       static_cast<const T*>(C), static_cast<const T*>(dt), A, states, states_b, R, L, H, P, N, G,
                       (int)s.Q, s.nC);
    BWD_CHECK(hipGetLastError());
    hipLaunchKernelGGL(finish_kernel<T>, dim3((unsigned)H, (unsigned)b), dim3(256), 0, st, q, R, dxy,
                       static_cast<const T*>(dt), A, static_cast<T*>(ddt), dA_part, dD_part, L, H);
    BWD_CHECK(hipGetLastError());
    hipLaunchKernelGGL(reduce_kernel, grid1(H), dim3(256), 0, st, dA_part, dD_part, dA, dD, b, H);
    BWD_CHECK(hipGetLastError());
    if (dh0) {
        hipLaunchKernelGGL(dh0_kernel<T>, grid1(b * H * PN), dim3(256), 0, st, G0, static_cast<const T*>(dt), A,
                           dfinal, dh0, L, H, PN, b * H * PN);
        BWD_CHECK(hipGetLastError());
    }
#undef BWD_CHECK
    return hipSuccess;
}

}  // namespace bwd

// Chunk of the transposed scans of the local flow, run as (N / 64) H heads of headdim and dstate 64: the
// forward's rule for that shape, at least the backward's chunk (so their states fit the space of its
// chunk states).
static int64_t transposed_chunk(const Shape& s) {
    Shape h = s;
    h.H = s.N / 64 * s.H;
    h.P = 64;
    h.N = 64;
    h.G = s.H;
    const int64_t q = fast_forward_chunk(h);
    return q < s.Q ? s.Q : q;
}

BackwardLayout backward_layout(const Shape& s) {
    auto a256 = [](size_t v) { return (v + 255) / 256 * 256; };
    BackwardLayout f{};
    f.local = decay_grad_supported(s);
    f.Lr = s.nC * s.Q;  // the reversed walks: front-padded to whole chunks
    const size_t BLHN = (size_t)(s.b * s.L * s.H * s.N) * 4, BLH = (size_t)(s.b * s.L * s.H) * 4;
    const size_t CS = (size_t)(s.b * s.H * s.nC * s.Q) * 4, ST = (size_t)(s.b * s.nC * s.H * s.P * s.N) * 4;
    const size_t HS = (size_t)(s.b * s.H * s.P * s.N) * 4, BH8 = (size_t)(s.b * s.H) * 8;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += a256(bytes);
        return at;
    };
    if (f.local) {
        // the stored states at the backward's chunk Q, the scans' bf16 outputs v and w (forward time), the
        // transposed final states, per-token q, dy.x and R, per-tile partial sums
        if (quad_combine(s)) {
            // the combine runs in halves, so w (read for dC before (c) runs), then v (read for dB before (b)
            // runs), then the adjoint's states take turns in one region
            f.states = take(ST);
            f.v_r = f.w = f.states_b = take(std::max(ST, BLHN / 2));
        } else {
            f.states = take(ST), f.states_b = take(ST);
            f.v_r = take(BLHN / 2), f.w = take(BLHN / 2);
        }
        f.G0 = take(HS), f.dfT = take(HS), f.h0T = take(HS), f.finT = take(HS);
        f.q = take(BLH), f.dxy = take(BLH), f.R = take(BLH);
        const size_t PART = (size_t)(s.b * ((s.L + 31) / 32) * s.H) * 8;
        f.dA_part = take(PART), f.dD_part = take(PART);
        // the large-chunk scans: sub-chunk-local decay arrays (reversed per head and per half-head, forwards
        // per half-head and per head), chunk totals and chunk-start states (transposed, per half-head)
        f.Qt = transposed_chunk(s);
        const int64_t nh = s.N / 64, H2 = nh * s.H, nsr = f.Lr / 64, nsf = (s.L + 63) / 64;
        const int64_t heads_r = s.H + (nh == 2 ? H2 : 0), heads_f = H2;
        f.sub = take((size_t)(2 * s.b * 64 * (heads_r * nsr + heads_f * nsf)) * 4);
        const int64_t nct = (f.Lr + f.Qt - 1) / f.Qt;  // at least the forward chunk count (L <= Lr)
        f.totals = take((size_t)(s.b * H2 * nct) * 4);
        f.stT = take((size_t)(s.b * nct * s.H * s.N * s.P) * 4);
        f.cbt = take(decay_grad_tile_bytes(s));  // the chunks' C . B tiles
    } else {
        const size_t sz = s.io == 1 ? 2 : 4;  // the reversed copies keep the input dtype
        const size_t RLHP = (size_t)(s.b * f.Lr * s.H * s.P) * 4, RLHN = (size_t)(s.b * f.Lr * s.H * s.N) * 4;
        const size_t RLGN = (size_t)(s.b * f.Lr * s.G * s.N), RLH = (size_t)(s.b * f.Lr * s.H) * 4;
        f.xr = take(RLHP / 4 * sz), f.dyr = take(RLHP / 4 * sz), f.Cr = take(RLGN * sz), f.Br = take(RLGN * sz);
        f.drev = take(RLH), f.dfwd = take(BLH), f.dt_t = take(CS), f.cs = take(CS), f.states = take(ST);
        f.u_r = take(RLHP), f.v_r = take(RLHN), f.w = take(BLHN), f.states_b = take(ST);
        f.G0 = take(HS), f.dfT = take(HS), f.h0T = take(HS), f.finT = take(HS), f.fscr = take(HS);
        f.q = take(BLH), f.dxy = take(BLH), f.R = take(BLH), f.dA_part = take(BH8), f.dD_part = take(BH8);
    }
    f.total = o;
    return f;
}

hipError_t launch_backward(const Shape& s, const void* x, const void* dt, const float* A, const void* B,
                           const void* C, const float* D, const float* h0, const void* dy, const float* dfinal,
                           void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, void* workspace,
                           hipStream_t st) {
    const BackwardLayout f = backward_layout(s);
    char* ws = static_cast<char*>(workspace);
    if (s.io == 1 && f.local && s.b > 0 && s.L > 0)
        return bwd::run_local(s, f, x, dt, A, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0, ws, st);
    if (s.io == 1)
        return bwd::run<bf16>(s, f, x, dt, A, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0, ws, st);
    return bwd::run<float>(s, f, x, dt, A, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0, ws, st);
}

}  // namespace ssd
