// chunk_state.hip -- chunk-local states from a zero start.
//
// First half of the state kernel on the devotd.net cuTile Mamba-2 page
// (section 2).  Unrolling the recurrence over one chunk gives
//     s_c[p, n] = sum_j w_j x_j[p] B_j[n],   w_j = 2^(l[Q-1] - l[j]) dt_j,
// one contraction over the chunk's tokens per (b, c, h).  The decay factor is
// fp32 and never exceeds 1 (the exponent is <= 0 for A <= 0).
//
// Workgroup = 4 wavefronts for one (b, c, h, N-block).  Tokens are staged in
// LDS in slices of 64, transposed so that each MFMA operand is a single 16-byte
// LDS read along the token axis.  For bf16 inputs the scaled operand w_j x_j
// is split into hi + lo bf16 parts and both are multiplied by the exact bf16
// B: the chunk state then carries ~2^-17 relative error instead of the ~2^-9
// of one bf16 rounding, which the final state needs.  fp32 compute uses fp32
// MFMA (16x16x4) and needs no split; its inputs may be fp32 or bf16 (I).
// Heads may share their x rows: head h reads x head h / xrep (xrep = 1: its own).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kCsSlice = 64;           // tokens per LDS slice
constexpr int kCsRow = kCsSlice + 8;   // padded LDS row, elements
constexpr int kCsMaxTiles = 16;        // 16x16 output tiles per wavefront

static inline int cs_nblock(int P, int N) {
    const int cand[4] = {128, 64, 32, 16};
    for (int nb : cand)
        if (N % nb == 0 && P * nb <= 16 * 16 * 4 * kCsMaxTiles) return nb;
    return 16;
}

template <class T>
static inline size_t cs_lds_bytes(int P, int Q, int NB) {
    constexpr bool kSplit = std::is_same<T, bf16>::value;
    size_t w = ((size_t)Q * 4 + 15) / 16 * 16;
    return w + (kSplit ? 2 : 1) * (size_t)P * kCsRow * sizeof(T) + (size_t)NB * kCsRow * sizeof(T);
}

template <class T, class I>
__global__ void __launch_bounds__(256) chunk_state_kernel(const I* __restrict__ x, const I* __restrict__ B,
                                                          const float* __restrict__ dt_t,
                                                          const float* __restrict__ cs, float* __restrict__ states,
                                                          int64_t L, int H, int P, int N, int G, int Q, int64_t nC,
                                                          int NB, int xrep, uint32_t nitems) {
    constexpr bool kSplit = std::is_same<T, bf16>::value;
    extern __shared__ __align__(16) unsigned char smem[];
    float* w = reinterpret_cast<float*>(smem);
    T* xh = reinterpret_cast<T*>(smem + ((size_t)Q * 4 + 15) / 16 * 16);
    T* xl = xh + (kSplit ? P * kCsRow : 0);
    T* bt = xl + P * kCsRow;

    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int nblocks = N / NB;
    const int h = (int)(item % H);
    const int nb = (int)((item / H) % nblocks);
    const int64_t c = (item / ((uint32_t)H * nblocks)) % nC;
    const int64_t b = item / ((uint32_t)H * nblocks * (uint32_t)nC);
    const int g = h / (H / G);
    const int Hx = H / xrep, hx = h / xrep;  // x rows of this head
    const int64_t cq = c * Q;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const float* csr = cs + ((b * H + h) * nC + c) * Q;
    const float* dtr = dt_t + ((b * H + h) * nC + c) * Q;
    const float lend = csr[Q - 1];
    for (int j = tid; j < Q; j += 256) w[j] = fast_exp2(lend - csr[j]) * dtr[j];

    const int tp = P / 16, tn = NB / 16, ntiles = tp * tn;
    f32x4 acc[kCsMaxTiles];
#pragma unroll
    for (int t = 0; t < kCsMaxTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j0 = 0; j0 < Q; j0 += kCsSlice) {
        const int klen = min(kCsSlice, Q - j0);
        const int kpad = (klen + 31) / 32 * 32;
        __syncthreads();
        // x^T slice, scaled by w_j (hi/lo split for bf16)
        const int p8n = P / 8;
        for (int task = tid; task < kpad * p8n; task += 256) {
            const int jj = task / p8n, p8 = (task % p8n) * 8;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const int64_t t = cq + j0 + jj;
            if (jj < klen && t < L) {
                load8_f32(x + ((b * L + t) * Hx + hx) * P + p8, v);
                const float wj = w[j0 + jj];
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] *= wj;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const T hi = from_f32<T>(v[q]);
                xh[(p8 + q) * kCsRow + jj] = hi;
                if (kSplit) xl[(p8 + q) * kCsRow + jj] = from_f32<T>(v[q] - to_f32(hi));
            }
        }
        // B^T slice
        const int n8n = NB / 8;
        for (int task = tid; task < kpad * n8n; task += 256) {
            const int jj = task / n8n, n8 = (task % n8n) * 8;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const int64_t t = cq + j0 + jj;
            if (jj < klen && t < L) load8_f32(B + ((b * L + t) * G + g) * N + (int64_t)nb * NB + n8, v);
#pragma unroll
            for (int q = 0; q < 8; ++q) bt[(n8 + q) * kCsRow + jj] = from_f32<T>(v[q]);
        }
        __syncthreads();
        for (int ks = 0; ks < kpad; ks += 32) {
#pragma unroll
            for (int tt = 0; tt < kCsMaxTiles; ++tt) {
                const int tile = wave + 4 * tt;
                if (tile < ntiles) {
                    const int pt = tile / tn, nt = tile % tn;
                    Frag<T> a, bo;
                    frag_load8<T>(bo, bt + (nt * 16 + l16) * kCsRow + ks + 8 * g4);
                    frag_load8<T>(a, xh + (pt * 16 + l16) * kCsRow + ks + 8 * g4);
                    mma(acc[tt], a, bo);
                    if (kSplit) {
                        frag_load8<T>(a, xl + (pt * 16 + l16) * kCsRow + ks + 8 * g4);
                        mma(acc[tt], a, bo);
                    }
                }
            }
        }
    }
    float* out = states + ((b * nC + c) * H + h) * (int64_t)P * N;
#pragma unroll
    for (int tt = 0; tt < kCsMaxTiles; ++tt) {
        const int tile = wave + 4 * tt;
        if (tile < ntiles) {
            const int pt = tile / tn, nt = tile % tn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = pt * 16 + 4 * g4 + r;
                out[(int64_t)p * N + nb * NB + nt * 16 + l16] = acc[tt][r];
            }
        }
    }
}

size_t chunk_state_lds_bytes(const Shape& s) {
    const int NB = cs_nblock((int)s.P, (int)s.N);
    return s.io == 1 ? cs_lds_bytes<bf16>((int)s.P, (int)s.Q, NB) : cs_lds_bytes<float>((int)s.P, (int)s.Q, NB);
}

template <class T, class I>
static hipError_t launch_cs(const Shape& s, int xrep, const void* x, const void* B, const float* dt_t, const float* cs,
                            float* states, hipStream_t st) {
    const int NB = cs_nblock((int)s.P, (int)s.N);
    const uint32_t nitems = (uint32_t)(s.b * s.nC * s.H * (s.N / NB));
    if (nitems == 0) return hipSuccess;
    const size_t lds = cs_lds_bytes<T>((int)s.P, (int)s.Q, NB);
    hipError_t e = hipFuncSetAttribute((const void*)chunk_state_kernel<T, I>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_state_kernel<T, I>), dim3(nitems), dim3(256), lds, st, (const I*)x, (const I*)B, dt_t,
                       cs, states, s.L, (int)s.H, (int)s.P, (int)s.N, (int)s.G, (int)s.Q, s.nC, NB, xrep, nitems);
    return hipGetLastError();
}

hipError_t launch_chunk_state_in(const Shape& s, int in_io, int xrep, const void* x, const void* B,
                                 const float* dt_t, const float* cs, float* states, hipStream_t st) {
    if (s.io == 1) return in_io == 1 ? launch_cs<bf16, bf16>(s, xrep, x, B, dt_t, cs, states, st) : hipErrorInvalidValue;
    return in_io == 1 ? launch_cs<float, bf16>(s, xrep, x, B, dt_t, cs, states, st)
                      : launch_cs<float, float>(s, xrep, x, B, dt_t, cs, states, st);
}

hipError_t launch_chunk_state(const Shape& s, const void* x, const void* B, const float* dt_t, const float* cs,
                              float* states, hipStream_t st) {
    if (fast_chunk_supported(s)) return launch_chunk_state_fast(s, x, B, dt_t, cs, states, st);
    return launch_chunk_state_in(s, s.io, 1, x, B, dt_t, cs, states, st);
}

}  // namespace ssd
