// decay_grad.hip -- the backward's decay gradient, chunk by chunk.
//
// The loss depends on the log-decay only through differences, so its gradient
// at token k is R_k = sum_{t>=k} dlambda_t, and the identity
//     R_k = a_k <G_k, S_{k-1}>                (a_k = 2^(dt_k A log2 e))
// with S the forward state and G the adjoint ("3.3 Hardware-Aware algorithms
// and GPU memory hierarchy optimisation", section 6: the backward recomputes
// states instead of storing them) turns that long suffix sum, whose terms
// nearly cancel over the whole sequence, into a sum of chunk-local terms.  With
// S0 the forward state entering chunk [c0, c1], Gam the adjoint entering it from
// the next chunk (a_{c1+1} G_{c1+1}; dfinal for the last chunk) and l the
// in-chunk cumulative log2 decay:
//   T1   = 2^(l_c1) <Gam, S0>                                   (one per chunk)
//   T2_k = sum_{t>=k} 2^(l_t) dy_t . (S0 C_t)                    (suffix sum)
//   T3_k = sum_{j<k} dt_j 2^(l_c1 - l_j) x_j . (Gam B_j)         (prefix sum)
//   T4_k = sum_{t>=k>j} M_tj,  M_tj = (dy_t . x_j)(C_t . B_j) 2^(l_t - l_j) dt_j
//   R_k  = T1 + T2_k + T3_k + T4_k
// (substituting both chunk-local expansions into a_k <G_k, S_{k-1}>; the
// decays combine as a_k 2^(l_{k-1}) = 2^(l_k)).  T4 follows from the column and
// row sums of the strictly lower triangle of M: T4_{k+1} = T4_k + colsum_k -
// rowsum_k.  Each term is accurate relative to itself, so the decay gradient
// no longer needs fp32 scans: dy . x and C . B are exact bf16 products with
// fp32 accumulation, and S0 and Gam enter the MFMA split into hi + lo bf16.
//
// T4's C . B factor does not depend on the head: a small kernel forms its tiles once per (b, chunk, group)
// and every head of the group reads them.  The per-head kernel then keeps only x, dy and one B-or-C tile
// in LDS (under half of a CU's), so two of its workgroups share each CU.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace dg {

constexpr int P = 64;
constexpr int QMAX = 128;
constexpr int XS = P + 8;  // x / dy row stride (bf16): 16-byte fragment reads of 16 rows hit distinct banks

// tiles on and below the diagonal of a chunk's Q x Q matrix, 16 x 16 each
__host__ __device__ constexpr int tri_tiles(int Q) { return (Q / 16) * (Q / 16 + 1) / 2; }

// column-major order of those tiles: column jt holds rows it = jt .. QT - 1 and starts at tile col_start(jt)
__host__ __device__ constexpr int col_start(int QT, int jt) { return jt * QT - jt * (jt - 1) / 2; }

// tile k -> (it, jt)
__device__ __forceinline__ void col_index(int k, int QT, int& it, int& jt) {
    jt = 0;
    while (col_start(QT, jt + 1) <= k) ++jt;
    it = jt + (k - col_start(QT, jt));
}

// a buffer resource over rows [0, rows) of a row-major bf16 tile (row_stride elements apart, row_len
// elements read per row); rows past it read zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* base, int64_t row_stride, int rows,
                                                           int row_len) {
    const int bytes = rows > 0 ? (int)(((int64_t)(rows - 1) * row_stride + row_len) * 2) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ldr(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 8 fp32 values -> hi and lo bf16 fragments
__device__ __forceinline__ void split8(const float4& a, const float4& b, Frag<bf16>& hi, Frag<bf16>& lo) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const bf16 h = static_cast<bf16>(v[s]);
        hi.v[s] = h;
        lo.v[s] = static_cast<bf16>(v[s] - static_cast<float>(h));
    }
}

// C_t . B_j over the tiles on and below the diagonal of each (b, chunk, group), as exact bf16 products
// with fp32 accumulation.  cbt: (b, nC, G, tri_tiles(Q), 256) fp32, tiles in column-major order (col_index),
// each in the accumulator order: float 4 l + r of tile (it, jt) is row 16 it + 4 (l / 16) + r, column
// 16 jt + l % 16 (rows past the sequence end are zero).  One workgroup of four wavefronts per item; B and C of the chunk in LDS.
template <int N>
__global__ void __launch_bounds__(256) cb_tiles_kernel(const bf16* __restrict__ B, const bf16* __restrict__ C,
                                                       float* __restrict__ cbt, int64_t L, int G, int Q, int64_t nC,
                                                       uint32_t nitems) {
    constexpr int NK = N / 32, NS = N + 8;
    __shared__ bf16 bs[QMAX * NS];
    __shared__ bf16 cs[QMAX * NS];
    const uint32_t item = xcd_remap(blockIdx.x, nitems);  // (b nC + c) G + g
    const int g = (int)(item % (uint32_t)G);
    const int64_t c = (item / (uint32_t)G) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)G * (uint32_t)nC);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t c0 = c * Q, GN = (int64_t)G * N;
    const int valid = (int)(L - c0 < Q ? L - c0 : Q);
    const auto rb = rows_rsrc(B + ((b * L + c0) * G + g) * (int64_t)N, GN, valid, N);
    const auto rc = rows_rsrc(C + ((b * L + c0) * G + g) * (int64_t)N, GN, valid, N);
    constexpr int KB = QMAX * (N / 8) / 256, BR = 256 / (N / 8);  // pieces per thread; rows per pass
    const int r0 = tid / (N / 8), col = (tid % (N / 8)) * 8;
    uint4 vb[KB], vc[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const uint32_t off = (uint32_t)(((int64_t)(r0 + BR * k) * GN + col) * 2);
        vb[k] = ldr(rb, off);
        vc[k] = ldr(rc, off);
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        if (r0 + BR * k < Q) {
            *reinterpret_cast<uint4*>(&bs[(r0 + BR * k) * NS + col]) = vb[k];
            *reinterpret_cast<uint4*>(&cs[(r0 + BR * k) * NS + col]) = vc[k];
        }
    }
    __syncthreads();
    const int ntiles = tri_tiles(Q);
    float* out = cbt + (int64_t)item * ntiles * 256 + lane * 4;
    for (int k = w; k < ntiles; k += 4) {
        int it, jt;
        col_index(k, Q / 16, it, jt);
        f32x4 ac = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            Frag<bf16> a, bo;
            frag_load8<bf16>(a, &cs[(16 * it + l16) * NS + 32 * ks + 8 * g4]);
            frag_load8<bf16>(bo, &bs[(16 * jt + l16) * NS + 32 * ks + 8 * g4]);
            mma(ac, a, bo);
        }
        *reinterpret_cast<float4*>(out + k * 256) = make_float4(ac[0], ac[1], ac[2], ac[3]);
    }
}

template <int N>
struct alignas(16) Lds {
    static constexpr int NS = N + 8;  // B / C row stride (bf16)
    bf16 xs[QMAX * XS];
    bf16 ys[QMAX * XS];   // dy
    bf16 bc[QMAX * NS];   // C while T2 runs, then B for T3
    float lw[QMAX];       // in-chunk cumulative log2 decay (flat past the sequence end)
    float dtw[QMAX];      // dt (zero past the sequence end)
    float rowsum[QMAX];
    float colsum[QMAX];
    float s2[QMAX];       // dy_t . (S0 C_t), before the factor 2^(l_t)
    float s3[QMAX];       // x_j . (Gam B_j), before dt_j 2^(l_c1 - l_j)
    float red[4];
};

// T2 (C with S0, read out by dy) or T3 (B with Gam, read out by x) for the state rows p = 16 pt + l16 and
// the token tiles it = half, half + 2, ...: the sum over p of D_tp (St A_t)_p into out[t]
template <int N>
__device__ __forceinline__ void state_term(const bf16* A, const bf16* Dm, float* out, const Frag<bf16> (&sh)[N / 32],
                                           const Frag<bf16> (&sl)[N / 32], int pt, int half, int QT, int l16, int g4) {
    constexpr int NK = N / 32, NS = Lds<N>::NS;
    for (int it = half; it < QT; it += 2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            Frag<bf16> a;
            frag_load8<bf16>(a, &A[(16 * it + l16) * NS + 32 * ks + 8 * g4]);
            mma(acc, a, sh[ks]);
            mma(acc, a, sl[ks]);
        }
        // acc[r] = (St A_t)_p for t = 16 it + 4 g4 + r; the four sums over p land in lanes l16 = 4 r
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<float>(Dm[(16 * it + 4 * g4 + r) * XS + 16 * pt + l16]) * acc[r];
        const float vs = row16_sum4(v[0], v[1], v[2], v[3], l16);
        if ((l16 & 3) == 0) atomicAdd(&out[16 * it + 4 * g4 + (l16 >> 2)], vs);
    }
}

// R and dxy (dy_t . x_t, for dD) (b, H, L) fp32.  dt (b, L, H) bf16 and A give the chunk's decays: dt of
// each token (zero past L) and the in-chunk cumulative log2 decay, from a wavefront scan of dt A per 64
// tokens (at chunk 128 the second wavefront adds the first's total once both are in LDS); cbt:
// cb_tiles_kernel's C . B tiles; S0: forward chunk-start states
// (b, nC, H, P, N); Gst: the reversed adjoint scan's chunk-start states (b, nC, H, P, N) in reversed chunk
// order, so forward chunk c reads reversed chunk nC - 1 - c: the adjoint G_{c1+1} of the token after the
// chunk (dfinal for the last chunk), which enters decayed by that token's factor 2^(cs of the next chunk's
// first position).
//
// Eight wavefronts; wavefront w holds rows 16 (w % 4) .. + 15 of both S0 and Gam in registers (hi + lo
// bf16 fragments, read once) and forms T2, then T3, for those 16 of the P output columns over every other
// 16-token tile of the chunk (w / 4 picks which); the parts of each term meet in LDS.  x and dy of the
// chunk sit in LDS, and one tile that holds C for T2 and is then refilled with B for T3.  All eight share
// the tiles of M, whose C . B factor comes from cbt.
template <int N>
__global__ void __launch_bounds__(512) decay_grad_kernel(const bf16* __restrict__ x, const bf16* __restrict__ dy,
                                                         const bf16* __restrict__ B, const bf16* __restrict__ C,
                                                         const bf16* __restrict__ dt,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ cbt,
                                                         const float* __restrict__ S0,
                                                         const float* __restrict__ Gst, float* __restrict__ R,
                                                         float* __restrict__ dxy, int64_t L, int H, int G, int Q,
                                                         int64_t nC, uint32_t nitems) {
    constexpr int NK = N / 32, NS = Lds<N>::NS;
    __shared__ Lds<N> sm;
    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int h = (int)(item % (uint32_t)H);
    const int64_t c = (item / (uint32_t)H) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)H * (uint32_t)nC);
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pt = w & 3;    // this wavefront's 16 state rows
    const int half = w >> 2; // its token tiles in T2 and T3
    const int QT = Q / 16;
    const int64_t c0 = c * Q;
    const int valid = (int)(L - c0 < Q ? L - c0 : Q);  // tokens of this chunk inside the sequence

    // ---- loads: x, dy and C pieces into LDS, B pieces held for T3 (zero past the sequence end), this
    // wavefront's rows of S0 and Gam ----------------------------------------------------------------------
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N;
    const auto rx = rows_rsrc(x + ((b * L + c0) * H + h) * (int64_t)P, HP, valid, P);
    const auto ry = rows_rsrc(dy + ((b * L + c0) * H + h) * (int64_t)P, HP, valid, P);
    const auto rb = rows_rsrc(B + ((b * L + c0) * G + g) * (int64_t)N, GN, valid, N);
    const auto rc = rows_rsrc(C + ((b * L + c0) * G + g) * (int64_t)N, GN, valid, N);
    constexpr int KX = QMAX * (P / 8) / 512, KB = QMAX * (N / 8) / 512;  // pieces per thread, largest chunk
    uint4 vx[KX], vy[KX], vb[KB], vc[KB];
    const int xr0 = tid >> 3, xc = (tid & 7) * 8;
    const int br0 = tid / (N / 8), bc = (tid % (N / 8)) * 8;
    constexpr int BR = 512 / (N / 8);  // B rows per pass of 512 threads
#pragma unroll
    for (int k = 0; k < KX; ++k) {
        const uint32_t off = (uint32_t)(((int64_t)(xr0 + 64 * k) * HP + xc) * 2);
        vx[k] = ldr(rx, off);
        vy[k] = ldr(ry, off);
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) vc[k] = ldr(rc, (uint32_t)(((int64_t)(br0 + BR * k) * GN + bc) * 2));
    const float* S0c = S0 + ((b * nC + c) * H + h) * (int64_t)P * N + (int64_t)(16 * pt + l16) * N + 8 * g4;
    const float* Gc = Gst + ((b * nC + (nC - 1 - c)) * H + h) * (int64_t)P * N + (int64_t)(16 * pt + l16) * N + 8 * g4;
    float4 sa[NK][2], ga[NK][2];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        sa[ks][0] = *reinterpret_cast<const float4*>(S0c + 32 * ks);
        sa[ks][1] = *reinterpret_cast<const float4*>(S0c + 32 * ks + 4);
        ga[ks][0] = *reinterpret_cast<const float4*>(Gc + 32 * ks);
        ga[ks][1] = *reinterpret_cast<const float4*>(Gc + 32 * ks + 4);
    }
    const float ah = A[h];
    if (tid < Q) {  // whole wavefronts (Q is 64 or 128)
        const float dv = c0 + tid < L ? static_cast<float>(dt[(b * L + c0 + tid) * H + h]) : 0.0f;
        sm.lw[tid] = wave_incl_scan(dv * ah) * kLog2e;  // the second wavefront's part still lacks the first's total
        sm.dtw[tid] = dv;
        sm.rowsum[tid] = 0.0f;
        sm.colsum[tid] = 0.0f;
        sm.s2[tid] = 0.0f;
        sm.s3[tid] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KX; ++k) {
        if (xr0 + 64 * k < Q) {
            *reinterpret_cast<uint4*>(&sm.xs[(xr0 + 64 * k) * XS + xc]) = vx[k];
            *reinterpret_cast<uint4*>(&sm.ys[(xr0 + 64 * k) * XS + xc]) = vy[k];
        }
    }
#pragma unroll
    for (int k = 0; k < KB; ++k)
        if (br0 + BR * k < Q) *reinterpret_cast<uint4*>(&sm.bc[(br0 + BR * k) * NS + bc]) = vc[k];
#pragma unroll
    for (int k = 0; k < KB; ++k) vb[k] = ldr(rb, (uint32_t)(((int64_t)(br0 + BR * k) * GN + bc) * 2));
    // T1 part: <S0, Gam> over this wavefront's rows (one wavefront per row block)
    if (half == 0) {
        float dot = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            const float4 v0 = ga[ks][0], v1 = ga[ks][1], u0 = sa[ks][0], u1 = sa[ks][1];
            dot = fmaf(u0.x, v0.x, fmaf(u0.y, v0.y, fmaf(u0.z, v0.z, fmaf(u0.w, v0.w, dot))));
            dot = fmaf(u1.x, v1.x, fmaf(u1.y, v1.y, fmaf(u1.z, v1.z, fmaf(u1.w, v1.w, dot))));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
        if (lane == 0) sm.red[pt] = dot;
    }
    Frag<bf16> sh[NK], sl[NK], gh[NK], gl[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        split8(sa[ks][0], sa[ks][1], sh[ks], sl[ks]);
        split8(ga[ks][0], ga[ks][1], gh[ks], gl[ks]);
    }
    __syncthreads();
    if (w == 1 && tid < Q) sm.lw[tid] += sm.lw[63];  // read again only after the barriers before T4

    // ---- dy_t . x_t per token (for dD): four threads per token, 16 columns each -------------------
    if (tid < 4 * Q) {
        const int t = tid >> 2, p0 = (tid & 3) * 16;
        float sxy = 0.0f;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.ys[t * XS + p0 + 8 * h8]);
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(&sm.xs[t * XS + p0 + 8 * h8]);
#pragma unroll
            for (int e = 0; e < 8; ++e) sxy = fmaf(static_cast<float>(a[e]), static_cast<float>(v[e]), sxy);
        }
        sxy = dpp_add<0xB1>(sxy);  // the four threads of the token: quad_perm [1,0,3,2], then [2,3,0,1]
        sxy = dpp_add<0x4E>(sxy);
        if ((tid & 3) == 0 && t < valid) dxy[(b * H + h) * L + c0 + t] = sxy;
    }

    // ---- T2 from the C tile; then the tile is refilled with B and T3 formed --------------------------
    state_term<N>(sm.bc, sm.ys, sm.s2, sh, sl, pt, half, QT, l16, g4);
    // this wavefront's run of C . B tiles of M (tiles k0 .. k1 - 1 in column-major order), fetched while
    // T3 runs into the registers that S0's fragments held
    const int ntiles = tri_tiles(Q);
    const int k0 = w * ntiles / 8, k1 = (w + 1) * ntiles / 8;
    const float* cbi = cbt + (((b * nC + c) * G + g) * (int64_t)ntiles + k0) * 256 + lane * 4;
    constexpr int KT = (tri_tiles(QMAX) + 7) / 8;
    float4 cbv[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k)
        cbv[k] = k0 + k < k1 ? *reinterpret_cast<const float4*>(cbi + k * 256) : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KB; ++k)
        if (br0 + BR * k < Q) *reinterpret_cast<uint4*>(&sm.bc[(br0 + BR * k) * NS + bc]) = vb[k];
    __syncthreads();
    state_term<N>(sm.bc, sm.xs, sm.s3, gh, gl, pt, half, QT, l16, g4);

    // ---- T4: the strictly lower triangle of M, tile by tile, into row and column sums.  Down a column of
    // tiles the x fragments, the column's decay and dt stay in registers and the column sums accumulate
    // there; each tile's four row sums take one LDS atomic. ------------------------------------------------
    {
        int jt = -1;
        Frag<bf16> xf[P / 32];
        float lj = 0.0f, dj = 0.0f, colp = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            const int k = k0 + kk;
            if (k >= k1) break;
            int it, jn;
            col_index(k, QT, it, jn);
            if (jn != jt) {
                if (jt >= 0) {
                    colp += __shfl_xor(colp, 16, 64);
                    colp += __shfl_xor(colp, 32, 64);
                    if (g4 == 0) atomicAdd(&sm.colsum[16 * jt + l16], colp);
                }
                jt = jn;
#pragma unroll
                for (int ks = 0; ks < P / 32; ++ks) frag_load8<bf16>(xf[ks], &sm.xs[(16 * jt + l16) * XS + 32 * ks + 8 * g4]);
                lj = sm.lw[16 * jt + l16];
                dj = sm.dtw[16 * jt + l16];
                colp = 0.0f;
            }
            f32x4 ad = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < P / 32; ++ks) {
                Frag<bf16> a;
                frag_load8<bf16>(a, &sm.ys[(16 * it + l16) * XS + 32 * ks + 8 * g4]);
                mma(ad, a, xf[ks]);
            }
            const float4 cb = cbv[kk];
            const float4 lt = *reinterpret_cast<const float4*>(&sm.lw[16 * it + 4 * g4]);
            const float ac[4] = {cb.x, cb.y, cb.z, cb.w}, lr[4] = {lt.x, lt.y, lt.z, lt.w};
            const int j = 16 * jt + l16;
            float m[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // j < t only; the exponent is capped at 0 so no masked lane forms an infinity
                m[r] = j < 16 * it + 4 * g4 + r ? ad[r] * ac[r] * fast_exp2(fminf(lr[r] - lj, 0.0f)) * dj : 0.0f;
                colp += m[r];
            }
            const float rs = row16_sum4(m[0], m[1], m[2], m[3], l16);  // row t = 16 it + 4 g4 + l16 / 4
            if ((l16 & 3) == 0) atomicAdd(&sm.rowsum[16 * it + 4 * g4 + (l16 >> 2)], rs);
        }
        if (jt >= 0) {
            colp += __shfl_xor(colp, 16, 64);
            colp += __shfl_xor(colp, 32, 64);
            if (g4 == 0) atomicAdd(&sm.colsum[16 * jt + l16], colp);
        }
    }
    __syncthreads();

    // ---- R_k = T1 + T2_k + T3_k + T4_k: one wavefront, two positions per lane ---------------------
    if (w == 0) {
        const float lend = sm.lw[Q - 1];
        // the adjoint enters decayed by the next token's factor (none after the sequence's end)
        const float gam = c + 1 < nC ? fast_exp2(static_cast<float>(dt[(b * L + c0 + Q) * H + h]) * ah * kLog2e) : 1.0f;
        const float T1 = fast_exp2(lend) * gam * (sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3]);
        float a2[2], a3[2], a4[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = 2 * lane + q;
            const bool in = k < Q;
            a2[q] = in ? fast_exp2(sm.lw[k]) * sm.s2[k] : 0.0f;
            a3[q] = in ? sm.dtw[k] * fast_exp2(lend - sm.lw[k]) * gam * sm.s3[k] : 0.0f;
            a4[q] = in ? sm.colsum[k] - sm.rowsum[k] : 0.0f;
        }
        // inclusive prefix sums over k of the pair sums, then per position
        const float p2 = wave_incl_scan(a2[0] + a2[1]), p3 = wave_incl_scan(a3[0] + a3[1]);
        const float p4 = wave_incl_scan(a4[0] + a4[1]);
        const float tot2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p2), 63));  // the whole sum
        // exclusive prefix before this lane's pair
        const float e2 = p2 - (a2[0] + a2[1]), e3 = p3 - (a3[0] + a3[1]), e4 = p4 - (a4[0] + a4[1]);
        float* Rh = R + (b * H + h) * L + c0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = 2 * lane + q;
            // T2_k: suffix from k = total - prefix before k; T3_k, T4_k: prefix before k
            const float pre2 = e2 + (q ? a2[0] : 0.0f), pre3 = e3 + (q ? a3[0] : 0.0f), pre4 = e4 + (q ? a4[0] : 0.0f);
            if (k < valid) Rh[k] = T1 + (tot2 - pre2) + pre3 + pre4;
        }
    }
}

}  // namespace dg

bool decay_grad_supported(const Shape& s) {
    return s.io == 1 && s.P == 64 && (s.N == 64 || s.N == 128) && (s.Q == 64 || s.Q == dg::QMAX);
}

size_t decay_grad_tile_bytes(const Shape& s) {
    return (size_t)(s.b * s.nC * s.G) * dg::tri_tiles((int)s.Q) * 256 * sizeof(float);
}

hipError_t launch_decay_grad(const Shape& s, const void* x, const void* dy, const void* B, const void* C,
                             const void* dt, const float* A, const float* S0, const float* Gst, float* cbt, float* R,
                             float* dxy, hipStream_t st) {
    const uint32_t nitems = (uint32_t)(s.b * s.nC * s.H), ncb = (uint32_t)(s.b * s.nC * s.G);
    if (nitems == 0) return hipSuccess;
    const bf16 *xb = (const bf16*)x, *yb = (const bf16*)dy, *bb = (const bf16*)B, *cb = (const bf16*)C,
               *dtb = (const bf16*)dt;
    if (s.N == 128) {
        hipLaunchKernelGGL(dg::cb_tiles_kernel<128>, dim3(ncb), dim3(256), 0, st, bb, cb, cbt, s.L, (int)s.G, (int)s.Q,
                           s.nC, ncb);
        hipLaunchKernelGGL(dg::decay_grad_kernel<128>, dim3(nitems), dim3(512), 0, st, xb, yb, bb, cb, dtb, A, cbt,
                           S0, Gst, R, dxy, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems);
    } else {
        hipLaunchKernelGGL(dg::cb_tiles_kernel<64>, dim3(ncb), dim3(256), 0, st, bb, cb, cbt, s.L, (int)s.G, (int)s.Q,
                           s.nC, ncb);
        hipLaunchKernelGGL(dg::decay_grad_kernel<64>, dim3(nitems), dim3(512), 0, st, xb, yb, bb, cb, dtb, A, cbt,
                           S0, Gst, R, dxy, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems);
    }
    return hipGetLastError();
}

}  // namespace ssd
