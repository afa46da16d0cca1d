// chunk_scan.hip -- chunk output from the chunk-start state.
//
// Third kernel on the devotd.net cuTile Mamba-2 page (section 2): for i < Q in
// chunk c,
//     y_i = 2^(l_i) C_i . S_c  +  sum_{j<=i} (C_i . B_j) 2^(l_i - l_j) dt_j x_j  +  D_h x_i.
// Three contractions: C . S^T (Q x N by N x P), G = B . C^T per 64 x 64 block,
// and the decayed, masked G times X.  The in-chunk Q x Q matrix never leaves
// registers: each wavefront computes G^T tiles for its own 16 query rows and
// feeds them, decayed and rounded, straight back into the next MFMA as the A
// operand (the K-order of the G accumulator layout is reused for X, so no
// register shuffle or LDS round trip is needed).  Positions above the diagonal
// are selected to zero, never computed as 0 * 2^(+x) (the static mask of the
// "Compiler-First State Space Duality ..." summary, Methodology).
//
// Workgroup = 4 wavefronts for one (b, c, h).  The chunk is walked in 64-row
// query blocks (one 16-row tile per wavefront) and 64-row key blocks up to the
// diagonal; C, B and S are staged in LDS in 64-wide slices of N, so every N up
// to 1024 fits.  The inputs may be bf16 under fp32 compute (I), and heads may
// share their x rows: head h reads x head h / xrep.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kScBlk = 64;            // query / key block rows
constexpr int kScNs = 64;             // N slice
constexpr int kScRow = kScNs + 8;     // padded LDS row, elements
constexpr int kScMaxP = 16;           // P / 16 <= 16

template <class T>
static inline size_t sc_lds_bytes(int P, int Q) {
    size_t lw = (size_t)2 * Q * 4;
    lw = (lw + 15) / 16 * 16;
    const int xrows = P > kScBlk ? P : kScBlk;
    return lw + (size_t)2 * kScBlk * kScRow * sizeof(T) + (size_t)xrows * kScRow * sizeof(T);
}

// Stage rows [r0, r0 + kScBlk) x cols [n0, n0 + ns) of a (b, L, G, N) tensor into LDS (zero padded).
template <class T, class I>
__device__ __forceinline__ void stage_rows(T* dst, const I* __restrict__ src, int64_t b, int64_t L, int G, int g,
                                           int N, int64_t cq, int Q, int r0, int n0, int ns, int kpad, int tid) {
    const int n8n = kpad / 8;
    for (int task = tid; task < kScBlk * n8n; task += 256) {
        const int rr = task / n8n, n8 = (task % n8n) * 8;
        const int i = r0 + rr;
        const int64_t t = cq + i;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (i < Q && t < L && n8 < ns) load8_f32(src + ((b * L + t) * G + g) * N + n0 + n8, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) dst[rr * kScRow + n8 + q] = from_f32<T>(v[q]);
    }
}

template <class T, class I>
__global__ void __launch_bounds__(256) chunk_scan_kernel(const I* __restrict__ x, const I* __restrict__ B,
                                                         const I* __restrict__ C, const float* __restrict__ dt_t,
                                                         const float* __restrict__ cs,
                                                         const float* __restrict__ start,
                                                         const float* __restrict__ D, T* __restrict__ y, int64_t L,
                                                         int H, int P, int N, int G, int Q, int64_t nC,
                                                         int xrep, uint32_t nitems) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* lw = reinterpret_cast<float*>(smem);
    float* dw = lw + Q;
    T* Cs = reinterpret_cast<T*>(smem + ((size_t)2 * Q * 4 + 15) / 16 * 16);
    T* Bs = Cs + kScBlk * kScRow;
    T* Xs = Bs + kScBlk * kScRow;  // S slice during C.S^T, then x^T of the key block

    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int h = (int)(item % H);
    const int64_t c = (item / H) % nC;
    const int64_t b = item / ((uint32_t)H * (uint32_t)nC);
    const int g = h / (H / G);
    const int Hx = H / xrep, hx = h / xrep;  // x rows of this head
    const int64_t cq = c * Q;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int tp = P / 16;

    const float* csr = cs + ((b * H + h) * nC + c) * Q;
    const float* dtr = dt_t + ((b * H + h) * nC + c) * Q;
    for (int j = tid; j < Q; j += 256) {
        lw[j] = csr[j];
        dw[j] = dtr[j];
    }
    const float* Sg = start + ((b * nC + c) * H + h) * (int64_t)P * N;
    const float Dh = D ? D[h] : 0.0f;

    for (int I0 = 0; I0 < Q; I0 += kScBlk) {
        const bool act = I0 + 16 * wave < Q;
        f32x4 yacc[kScMaxP];
#pragma unroll
        for (int t = 0; t < kScMaxP; ++t) yacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ---- inter-chunk part: C_i . S_c^T -----------------------------------
        for (int n0 = 0; n0 < N; n0 += kScNs) {
            const int ns = min(kScNs, N - n0), kpad = (ns + 31) / 32 * 32;
            __syncthreads();
            stage_rows<T, I>(Cs, C, b, L, G, g, N, cq, Q, I0, n0, ns, kpad, tid);
            const int n8n = kpad / 8;
            for (int task = tid; task < P * n8n; task += 256) {
                const int p = task / n8n, n8 = (task % n8n) * 8;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    Xs[p * kScRow + n8 + q] = from_f32<T>(n8 + q < ns ? Sg[(int64_t)p * N + n0 + n8 + q] : 0.0f);
            }
            __syncthreads();
            if (act) {
                for (int ks = 0; ks < kpad; ks += 32) {
                    Frag<T> a;
                    frag_load8<T>(a, Cs + (16 * wave + l16) * kScRow + ks + 8 * g4);
#pragma unroll
                    for (int pt = 0; pt < kScMaxP; ++pt) {
                        if (pt < tp) {
                            Frag<T> bo;
                            frag_load8<T>(bo, Xs + (pt * 16 + l16) * kScRow + ks + 8 * g4);
                            mma(yacc[pt], a, bo);
                        }
                    }
                }
            }
        }
        if (act) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sc = fast_exp2(lw[I0 + 16 * wave + 4 * g4 + r]);
#pragma unroll
                for (int pt = 0; pt < kScMaxP; ++pt) yacc[pt][r] *= sc;
            }
        }

        // ---- in-chunk part: key blocks up to the diagonal -------------------------
        const int irow = I0 + 16 * wave + l16;  // this lane's query row as the A-operand row
        const float li = act ? lw[irow] : 0.0f;
        for (int J0 = 0; J0 <= I0; J0 += kScBlk) {
            f32x4 gacc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) gacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int n0 = 0; n0 < N; n0 += kScNs) {
                const int ns = min(kScNs, N - n0), kpad = (ns + 31) / 32 * 32;
                __syncthreads();
                stage_rows<T, I>(Cs, C, b, L, G, g, N, cq, Q, I0, n0, ns, kpad, tid);
                stage_rows<T, I>(Bs, B, b, L, G, g, N, cq, Q, J0, n0, ns, kpad, tid);
                __syncthreads();
                if (act) {
                    for (int ks = 0; ks < kpad; ks += 32) {
                        Frag<T> bo;
                        frag_load8<T>(bo, Cs + (16 * wave + l16) * kScRow + ks + 8 * g4);
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt) {
                            Frag<T> a;
                            frag_load8<T>(a, Bs + (jt * 16 + l16) * kScRow + ks + 8 * g4);
                            mma(gacc[jt], a, bo);
                        }
                    }
                }
            }
            // x^T of the key block
            __syncthreads();
            const int p8n = P / 8;
            for (int task = tid; task < kScBlk * p8n; task += 256) {
                const int jj = task / p8n, p8 = (task % p8n) * 8;
                const int j = J0 + jj;
                const int64_t t = cq + j;
                float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (j < Q && t < L) load8_f32(x + ((b * L + t) * Hx + hx) * P + p8, v);
#pragma unroll
                for (int q = 0; q < 8; ++q) Xs[(p8 + q) * kScRow + jj] = from_f32<T>(v[q]);
            }
            __syncthreads();
            if (act) {
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    Frag<T> a;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int jt = 2 * jp + half;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = J0 + jt * 16 + 4 * g4 + r;
                            float m = 0.0f;
                            if (j <= irow) m = gacc[jt][r] * fast_exp2(li - lw[j]) * dw[j];
                            frag_set<T>(a, half * 4 + r, m);
                        }
                    }
#pragma unroll
                    for (int pt = 0; pt < kScMaxP; ++pt) {
                        if (pt < tp) {
                            Frag<T> bo;
                            const T* row = Xs + (pt * 16 + l16) * kScRow;
                            frag_load4x2<T>(bo, row + (2 * jp) * 16 + 4 * g4, row + (2 * jp + 1) * 16 + 4 * g4);
                            mma(yacc[pt], a, bo);
                        }
                    }
                }
            }
        }

        // ---- skip term and store ---------------------------------------------------
        if (act) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = I0 + 16 * wave + 4 * g4 + r;
                const int64_t t = cq + i;
                if (t < L) {
                    const int64_t row = ((b * L + t) * H + h) * (int64_t)P;
                    const int64_t xrow = ((b * L + t) * Hx + hx) * (int64_t)P;
#pragma unroll
                    for (int pt = 0; pt < kScMaxP; ++pt) {
                        if (pt < tp) {
                            const int p = pt * 16 + l16;
                            float v = yacc[pt][r];
                            if (D) v += Dh * to_f32(x[xrow + p]);
                            y[row + p] = from_f32<T>(v);
                        }
                    }
                }
            }
        }
    }
}

size_t chunk_scan_lds_bytes(const Shape& s) {
    return s.io == 1 ? sc_lds_bytes<bf16>((int)s.P, (int)s.Q) : sc_lds_bytes<float>((int)s.P, (int)s.Q);
}

template <class T, class I>
static hipError_t launch_sc(const Shape& s, int xrep, const void* x, const void* B, const void* C, const float* dt_t,
                            const float* cs, const float* start, const float* D, void* y, hipStream_t st) {
    const uint32_t nitems = (uint32_t)(s.b * s.nC * s.H);
    if (nitems == 0) return hipSuccess;
    const size_t lds = sc_lds_bytes<T>((int)s.P, (int)s.Q);
    hipError_t e = hipFuncSetAttribute((const void*)chunk_scan_kernel<T, I>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_scan_kernel<T, I>), dim3(nitems), dim3(256), lds, st, (const I*)x, (const I*)B,
                       (const I*)C, dt_t, cs, start, D, (T*)y, s.L, (int)s.H, (int)s.P, (int)s.N, (int)s.G,
                       (int)s.Q, s.nC, xrep, nitems);
    return hipGetLastError();
}

hipError_t launch_chunk_scan_in(const Shape& s, int in_io, int xrep, const void* x, const void* B, const void* C,
                                const float* dt_t, const float* cs, const float* start, const float* D, void* y,
                                hipStream_t st) {
    if (s.io == 1)
        return in_io == 1 ? launch_sc<bf16, bf16>(s, xrep, x, B, C, dt_t, cs, start, D, y, st) : hipErrorInvalidValue;
    return in_io == 1 ? launch_sc<float, bf16>(s, xrep, x, B, C, dt_t, cs, start, D, y, st)
                      : launch_sc<float, float>(s, xrep, x, B, C, dt_t, cs, start, D, y, st);
}

hipError_t launch_chunk_scan(const Shape& s, const void* x, const void* B, const void* C, const float* dt_t,
                             const float* cs, const float* start, const float* D, void* y, hipStream_t st) {
    if (fast_chunk_supported(s)) return launch_chunk_scan_fast(s, x, B, C, dt_t, cs, start, D, y, st);
    return launch_chunk_scan_in(s, s.io, 1, x, B, C, dt_t, cs, start, D, y, st);
}

}  // namespace ssd
