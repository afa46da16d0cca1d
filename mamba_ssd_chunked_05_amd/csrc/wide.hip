// wide.hip -- chunk-state and chunk-scan kernels for a wide state: bf16 inputs,
// headdim 64, dstate 256 or 512, any chunk that is a multiple of 64.
//
// They compute the same staged calls as fused.hip (the chunk-local states and
// the chunk output from the chunk-start state, cuTile page on devotd.net,
// section 2), with the same 64-token sub-chunk walk: per sub-chunk
//   y  = 2^(l_i) C_i . S + sum_{j<=i} (C_i . B_j) 2^(l_i-l_j) dt_j x_j + D x_i
//   S <- 2^(l_63) S + sum_j 2^(l_63-l_j) dt_j B_j (outer) x_j.
// Every term is a sum over the state index n ("3.3 Hardware-Aware ...",
// section 4.1: the output through C is linear in the state), so a sub-chunk is
// processed in blocks of 128 state columns: the B and C tiles of one block sit
// in LDS at a time (the LDS footprint of dstate 128), the products over n
// accumulate across blocks in registers, and the state update of a block runs
// right after that block's part of C . S has read the old state.
//
// One head per workgroup.  chunk_state_wide_kernel and chunk_scan_wide_kernel
// (dstate 256) run four wavefronts; wavefront w carries the fp32 state rows
// p = 16w .. 16w + 15 for all N columns in registers (N/4 values per lane).
// chunk_scan_wide8_kernel (dstate 512) runs eight, each with one p-tile and
// one half of the state columns; chunk_state_wide32_kernel (dstate 512) holds
// the state transposed in 32 x 32 tiles for the 32 x 32 x 16 MFMA.
// Staging of the next block (or the next sub-chunk) runs one step ahead in
// registers.  Layout and fragment conventions are those of fused.hip.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ssd {
namespace fz {

constexpr int WB = 128;       // state columns per LDS block
constexpr int WBS = WB + 16;  // B block row stride (bf16): transpose reads
constexpr int WCS = WB + 8;   // C block row stride (bf16): row reads

// one head's sub-chunk staging: x (2 pieces), one B/C block (4 + 4 pieces), dt and cs
struct WideRegs {
    uint4 x[2];
    uint4 b[4];
    uint4 c[4];
    float dt, cs;
};

// Per-thread piece coordinates.  x: rows tid / 8 (+ 32), columns 8 (tid % 8);
// B / C block: rows tid / 16 (+ 16 k), columns 8 (tid % 16) of the block.
struct WideAddr {
    int xr, xc, br, bc;
    uint32_t xo, bo;  // byte offsets of the first x piece and of the B / C piece within their tiles
};

struct WideSrc {
    const bf16 *x, *B, *C;
    DtSrc ds;
    int64_t b, L, dt0;  // dt0: this chunk's first dt/cs element of the head
    int H, G, N, h, g;
};

// x, dt and cs of sub-chunk `sub` starting at token tbase
__device__ __forceinline__ void wide_load_x(WideRegs& rg, const WideAddr& a, const WideSrc& s, int64_t tbase, int sub,
                                            int tid) {
    const int64_t HP_ = (int64_t)s.H * P;
    const auto r = tile_rsrc(s.x + ((s.b * s.L + tbase) * s.H + s.h) * (int64_t)P, HP_, s.L - tbase, P);
#pragma unroll
    for (int k = 0; k < 2; ++k) rg.x[k] = ldbuf(r, a.xo + (uint32_t)(32 * k * HP_ * 2));
    if (tid < 64) {
        rg.dt = s.ds.dt_t[s.dt0 + (int64_t)QS * sub + tid];
        rg.cs = s.ds.cs[s.dt0 + (int64_t)QS * sub + tid];
    }
}

// block nb (columns 128 nb ..) of B (and C) for the sub-chunk starting at tbase
template <bool WITH_C>
__device__ __forceinline__ void wide_load_bc(WideRegs& rg, const WideAddr& a, const WideSrc& s, int64_t tbase, int nb) {
    const int64_t GN = (int64_t)s.G * s.N, off = ((s.b * s.L + tbase) * s.G + s.g) * (int64_t)s.N;
    const auto rb = tile_rsrc(s.B + off, GN, s.L - tbase, s.N);
    const auto rc = tile_rsrc(WITH_C ? s.C + off : s.B + off, GN, s.L - tbase, s.N);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t o = a.bo + (uint32_t)((16 * k * GN + WB * nb) * 2);
        rg.b[k] = ldbuf(rb, o);
        if (WITH_C) rg.c[k] = ldbuf(rc, o);
    }
}

template <bool WITH_C>
__device__ __forceinline__ void wide_store_bc(bf16* bsb, bf16* csb, const WideRegs& rg, const WideAddr& a) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        *reinterpret_cast<uint4*>(bsb + (a.br + 16 * k) * WBS + a.bc) = rg.b[k];
        if (WITH_C) *reinterpret_cast<uint4*>(csb + (a.br + 16 * k) * WCS + a.bc) = rg.c[k];
    }
}

// the decay vectors of the sub-chunk (wavefront 0, lane = token); see chunk_store in fused.hip
template <bool FWD>
__device__ __forceinline__ void wide_decay_store(float* lw, float* dtw, float* ww, float* ec, float* alpha, float dtv,
                                                 float csv, float& cs_prev, float& tot, int tid) {
    {
        const int lane = tid;
        const float d = dtv;
        float incl;
        if (FWD) {
            incl = csv;
        } else {
            incl = csv - cs_prev;
            cs_prev = __shfl(csv, 63, 64);
        }
        const float last = __shfl(incl, 63, 64);
        tot += last;
        lw[lane] = incl;
        dtw[lane] = d;
        ww[lane] = fast_exp2(last - incl) * d;
        if (ec) {
            ec[lane] = fast_exp2(incl - __shfl(incl, lane & ~15, 64));
#pragma unroll
            for (int it = 1; it < 4; ++it) ec[it * QS + lane] = fast_exp2(fminf(__shfl(incl, 16 * it, 64) - incl, 0.0f)) * d;
        }
        if (lane == 0) alpha[0] = fast_exp2(last);
    }
}

// x to LDS and the decay vectors of the sub-chunk (wavefront 0)
template <bool FWD>
__device__ __forceinline__ void wide_store_x(bf16* xs, float* lw, float* dtw, float* ww, float* ec, float* alpha,
                                             const WideRegs& rg, const WideAddr& a, float& cs_prev, float& tot,
                                             int tid) {
#pragma unroll
    for (int k = 0; k < 2; ++k) *reinterpret_cast<uint4*>(xs + (a.xr + 32 * k) * XS + a.xc) = rg.x[k];
    if (tid < 64) wide_decay_store<FWD>(lw, dtw, ww, ec, alpha, rg.dt, rg.cs, cs_prev, tot, tid);
}

__device__ __forceinline__ void wide_addr(WideAddr& a, const WideSrc& s, int tid) {
    a.xr = tid >> 3;
    a.xc = (tid & 7) * 8;
    a.br = tid >> 4;
    a.bc = (tid & 15) * 8;
    a.xo = (uint32_t)((a.xr * (int64_t)s.H * P + a.xc) * 2);
    a.bo = (uint32_t)((a.br * (int64_t)s.G * s.N + a.bc) * 2);
}

// ---------------------------------------------------------------------------
// chunk output
// ---------------------------------------------------------------------------
struct WideScanLds {
    bf16 xs[QS * XS];
    bf16 bs[QS * WBS];
    bf16 cs[QS * WCS];
    bf16 mb[16 * 256];  // decayed C.B^T tiles in fragment order [jt*4+it][lane][4]
    float lw[QS], dtw[QS], ww[QS];
    float ec[4 * QS];
    float alpha[4];
};

// dstate 512 keeps 128 state values per lane: one wavefront per SIMD, all registers
template <int N, bool FWD>
__global__ void __launch_bounds__(256, N >= 512 ? 1 : 2)
chunk_scan_wide_kernel(const bf16* __restrict__ x, const bf16* __restrict__ B, const bf16* __restrict__ C,
                       DtSrc ds, const float* __restrict__ start, const float* __restrict__ D, bf16* __restrict__ y,
                       int64_t L, int H, int G, int Q, int64_t nC, uint32_t nitems) {
    constexpr int NBLK = N / WB, NT = N / 16;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    WideScanLds& sm = *reinterpret_cast<WideScanLds*>(smem_raw);

    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int h = (int)(item % (uint32_t)H);
    const int64_t c = (item / (uint32_t)H) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)H * (uint32_t)nC);
    const int g = h / (H / G);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const float Dh = D ? D[h] : 0.0f;
    const int64_t t0 = c * Q;
    const int64_t t_end = t0 + Q < L ? t0 + Q : L;
    const int nsub = (int)((t_end - t0 + QS - 1) / QS);
    const int64_t nsubT = (L + QS - 1) / QS;
    float cs_prev = 0.0f, tot = 0.0f;

    // carried state, transposed: st[nt] holds S[p = 16w + l16][n = 16nt + 4g4 + r]
    f32x4 st[NT];
    {
        const float* S0 = start + ((b * nC + c) * H + h) * (int64_t)P * N + (int64_t)(16 * w + l16) * N + 4 * g4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st[nt] = *reinterpret_cast<const f32x4*>(S0 + 16 * nt);
    }
    // tiles above the diagonal that pair with a diagonal tile in a 32-wide K step stay zero
    sm.mb[(1 * 4 + 0) * 256 + tid] = static_cast<bf16>(0.0f);
    sm.mb[(3 * 4 + 2) * 256 + tid] = static_cast<bf16>(0.0f);

    WideSrc src;
    src.x = x, src.B = B, src.C = C, src.ds = ds, src.b = b, src.L = L, src.H = H, src.G = G, src.N = N, src.h = h,
    src.g = g;
    src.dt0 = FWD ? ((b * H + h) * nsubT + c * (Q / QS)) * QS : ((b * H + h) * nC + c) * Q;
    WideAddr ad;
    wide_addr(ad, src, tid);
    WideRegs rg;
    wide_load_x(rg, ad, src, t0, 0, tid);
    wide_load_bc<true>(rg, ad, src, t0, 0);

    for (int sc = 0; sc < nsub; ++sc) {
        const int64_t tbase = t0 + (int64_t)sc * QS;
        const bool more = sc + 1 < nsub;
        __syncthreads();  // the previous sub-chunk's readers are done with the LDS tiles
        wide_store_x<FWD>(sm.xs, sm.lw, sm.dtw, sm.ww, sm.ec, sm.alpha, rg, ad, cs_prev, tot, tid);
        wide_store_bc<true>(sm.bs, sm.cs, rg, ad);
        __syncthreads();
        if (more) wide_load_x(rg, ad, src, tbase + QS, sc + 1, tid);
        if (NBLK > 1)
            wide_load_bc<true>(rg, ad, src, tbase, 1);
        else if (more)
            wide_load_bc<true>(rg, ad, src, tbase + QS, 0);

        // decay-scaled X^T fragments (token slots 32ks + 4g4 + r, 32ks + 16 + 4g4 + r)
        Frag<bf16> xw[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            Frag<bf16> xf;
            xf.v = pack8(tr_read(sm.xs, 32 * ks + 4 * g4, 16 * w, XS, l16),
                         tr_read(sm.xs, 32 * ks + 16 + 4 * g4, 16 * w, XS, l16));
            const float* wv = &sm.ww[32 * ks + 4 * g4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                xw[ks].v[r] = static_cast<bf16>(static_cast<float>(xf.v[r]) * wv[r]);
                xw[ks].v[4 + r] = static_cast<bf16>(static_cast<float>(xf.v[4 + r]) * wv[16 + r]);
            }
        }
        const float alpha = sm.alpha[0];
        f32x4 acc[4], gacc[3];
#pragma unroll
        for (int it = 0; it < 4; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 3; ++q) gacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb) {
            if (nb > 0) {
                __syncthreads();  // every wavefront is done with the previous block
                wide_store_bc<true>(sm.bs, sm.cs, rg, ad);
                __syncthreads();
                if (nb + 1 < NBLK)
                    wide_load_bc<true>(rg, ad, src, tbase, nb + 1);
                else if (more)
                    wide_load_bc<true>(rg, ad, src, tbase + QS, 0);
            }
            // C.B^T over this block's 128 columns for this wavefront's tiles w, w + 4 (, w + 8)
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int tt = w + 4 * q;
                if (tt < 10) {
                    const int it = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
                    const int jt = tt - it * (it + 1) / 2;
#pragma unroll
                    for (int ks = 0; ks < WB / 32; ++ks) {
                        Frag<bf16> a, bo;
                        frag_load8<bf16>(a, &sm.bs[(16 * jt + l16) * WBS + 32 * ks + 8 * g4]);
                        frag_load8<bf16>(bo, &sm.cs[(16 * it + l16) * WCS + 32 * ks + 8 * g4]);
                        mma(gacc[q], a, bo);
                    }
                }
            }
            // S C^T over this block, from the state before this sub-chunk's update
#pragma unroll
            for (int ks = 0; ks < WB / 32; ++ks) {
                Frag<bf16> sa;
                sa.v = pack8(cvt4(st[nb * (WB / 16) + 2 * ks]), cvt4(st[nb * (WB / 16) + 2 * ks + 1]));
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const bf16* crow = &sm.cs[(16 * it + l16) * WCS + 32 * ks];
                    Frag<bf16> bo;
                    bo.v = pack8(*reinterpret_cast<const bf16x4*>(crow + 4 * g4),
                                 *reinterpret_cast<const bf16x4*>(crow + 16 + 4 * g4));
                    mma(acc[it], sa, bo);
                }
            }
            // S <- 2^(l_63) S + B^T (w x) on this block's columns
#pragma unroll
            for (int nt = 0; nt < WB / 16; ++nt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) st[nb * (WB / 16) + nt][r] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int nt = 0; nt < WB / 16; ++nt) {
                    Frag<bf16> a;
                    a.v = pack8(tr_read(sm.bs, 32 * ks + 4 * g4, 16 * nt, WBS, l16),
                                tr_read(sm.bs, 32 * ks + 16 + 4 * g4, 16 * nt, WBS, l16));
                    mma(st[nb * (WB / 16) + nt], a, xw[ks]);
                }
            }
        }

        // decayed C.B^T tiles -> LDS (D_h on the diagonal, so X^T M also yields D x)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int tt = w + 4 * q;
            if (tt < 10) {
                const int it = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
                const int jt = tt - it * (it + 1) / 2;
                const int i = 16 * it + l16, j0 = 16 * jt + 4 * g4;
                f32x4 m;
                if (jt == it) {
                    const float li = sm.lw[i];
                    const f32x4 lj = *reinterpret_cast<const f32x4*>(&sm.lw[j0]);
                    const f32x4 dj = *reinterpret_cast<const f32x4*>(&sm.dtw[j0]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = gacc[q][r] * fast_exp2(fminf(li - lj[r], 0.0f)) * dj[r];
                        m[r] = (j0 + r <= i ? v : 0.0f) + (j0 + r == i ? Dh : 0.0f);
                    }
                } else {
                    const float er = sm.ec[i];
                    const f32x4 ej = *reinterpret_cast<const f32x4*>(&sm.ec[it * QS + j0]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[r] = gacc[q][r] * er * ej[r];
                }
                *reinterpret_cast<bf16x4*>(&sm.mb[((jt * 4 + it) * 64 + lane) * 4]) = cvt4(m);
            }
        }
        __syncthreads();

        // Y^T[p-tile w] = 2^l_i (S C^T) + X^T M
        const bool full = tbase + QS <= L;
        bf16* yb = y + ((b * L + tbase) * H + h) * (int64_t)P + 16 * w + 4 * g4;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = 16 * it + l16;
            const float sc_i = fast_exp2(sm.lw[i]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[it][r] *= sc_i;
#pragma unroll
            for (int js = 0; js <= it / 2; ++js) {
                Frag<bf16> a, bo;
                a.v = pack8(tr_read(sm.xs, 32 * js + 4 * g4, 16 * w, XS, l16),
                            tr_read(sm.xs, 32 * js + 16 + 4 * g4, 16 * w, XS, l16));
                bo.v = pack8(*reinterpret_cast<const bf16x4*>(&sm.mb[(((2 * js) * 4 + it) * 64 + lane) * 4]),
                             *reinterpret_cast<const bf16x4*>(&sm.mb[(((2 * js + 1) * 4 + it) * 64 + lane) * 4]));
                mma(acc[it], a, bo);
            }
            if (full || tbase + i < L) {
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[it][r]);
                *reinterpret_cast<bf16x4*>(yb + (int64_t)i * H * P) = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// chunk output with the state split over n: eight wavefronts, wavefront w owns
// p-tile w % 4 and state half w / 4 (columns (w / 4) N/2 ..).  Each pass stages
// one 128-column block of B and C for each half, so every B and C fragment is
// read only by the wavefronts of its half; the C.B^T tiles accumulate over both
// blocks of every pass.  The two halves' partial outputs C.S are exchanged
// through LDS at the end of the sub-chunk: half 0 finishes token tiles 0-1,
// half 1 token tiles 2-3.  Half the state per wavefront lets dstate 512 run two
// wavefronts per SIMD instead of one.
// ---------------------------------------------------------------------------
struct Wide8Lds {
    bf16 xs[QS * XS];
    bf16 bs[2][QS * WBS];  // per half: the pass's B block; reused for the partial-output exchange
    bf16 cs[2][QS * WCS];
    bf16 mb[16 * 256];
    float lw[QS], dtw[QS], ww[QS];
    float ec[4 * QS];
    float alpha[4];
};

struct Wide8Regs {
    uint4 x;
    uint4 b[4];
    uint4 c[4];
    float dt, cs;
};

// x of the sub-chunk at tbase (row tid / 8, columns 8 (tid % 8); byte offset xo), and its dt and cs
// (threads < 64)
__device__ __forceinline__ void wide8_load_x(Wide8Regs& rg, const WideSrc& s, int64_t tbase, int sub, int tid,
                                             uint32_t xo) {
    const auto r = tile_rsrc(s.x + ((s.b * s.L + tbase) * s.H + s.h) * (int64_t)P, (int64_t)s.H * P, s.L - tbase, P);
    rg.x = ldbuf(r, xo);
    if (tid < 64) {
        rg.dt = s.ds.dt_t[s.dt0 + (int64_t)QS * sub + tid];
        rg.cs = s.ds.cs[s.dt0 + (int64_t)QS * sub + tid];
    }
}

// pass q's two blocks of B and C: half tid / 256 takes columns (tid / 256) N/2 + 128 q ..,
// rows (tid % 256) / 16 + 16 k, columns 8 (tid % 16) of the block (byte offset bo for k = q = 0)
__device__ __forceinline__ void wide8_load_bc(Wide8Regs& rg, const WideSrc& s, int64_t tbase, int q, uint32_t bo) {
    const int64_t GN = (int64_t)s.G * s.N, off = ((s.b * s.L + tbase) * s.G + s.g) * (int64_t)s.N;
    const auto rb = tile_rsrc(s.B + off, GN, s.L - tbase, s.N);
    const auto rc = tile_rsrc(s.C + off, GN, s.L - tbase, s.N);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t o = bo + (uint32_t)((16 * k * GN + WB * q) * 2);
        rg.b[k] = ldbuf(rb, o);
        rg.c[k] = ldbuf(rc, o);
    }
}

__device__ __forceinline__ void wide8_store_bc(Wide8Lds& sm, const Wide8Regs& rg, int tid) {
    const int half = tid >> 8, r0 = (tid & 255) >> 4, cc = (tid & 15) * 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        *reinterpret_cast<uint4*>(&sm.bs[half][(r0 + 16 * k) * WBS + cc]) = rg.b[k];
        *reinterpret_cast<uint4*>(&sm.cs[half][(r0 + 16 * k) * WCS + cc]) = rg.c[k];
    }
}

// token tiles IT0, IT0 + 1 of the output: add the other half's partial C.S, scale by 2^l_i, add X^T M, store
template <int IT0>
__device__ __forceinline__ void wide8_finish(f32x4* acc, const Wide8Lds& sm, const float* px, int partner, int pt,
                                             int lane, int g4, int l16, bf16* yb, int64_t HP_, bool full,
                                             int64_t rows_left) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
        const int it = IT0 + o;
        const f32x4 pv = *reinterpret_cast<const f32x4*>(&px[((partner * 2 + o) * 64 + lane) * 4]);
        const int i = 16 * it + l16;
        const float sc_i = fast_exp2(sm.lw[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[it][r] = (acc[it][r] + pv[r]) * sc_i;
#pragma unroll
        for (int js = 0; js <= it / 2; ++js) {
            Frag<bf16> a, bo;
            a.v = pack8(tr_read(sm.xs, 32 * js + 4 * g4, 16 * pt, XS, l16),
                        tr_read(sm.xs, 32 * js + 16 + 4 * g4, 16 * pt, XS, l16));
            bo.v = pack8(*reinterpret_cast<const bf16x4*>(&sm.mb[(((2 * js) * 4 + it) * 64 + lane) * 4]),
                         *reinterpret_cast<const bf16x4*>(&sm.mb[(((2 * js + 1) * 4 + it) * 64 + lane) * 4]));
            mma(acc[it], a, bo);
        }
        if (full || i < rows_left) {
            bf16x4 ov;
#pragma unroll
            for (int r = 0; r < 4; ++r) ov[r] = static_cast<bf16>(acc[it][r]);
            *reinterpret_cast<bf16x4*>(yb + (int64_t)i * HP_) = ov;
        }
    }
}

template <int N, bool FWD>
__global__ void __launch_bounds__(512, 2)
chunk_scan_wide8_kernel(const bf16* __restrict__ x, const bf16* __restrict__ B, const bf16* __restrict__ C,
                        DtSrc ds, const float* __restrict__ start, const float* __restrict__ D,
                        bf16* __restrict__ y, int64_t L, int H, int G, int Q, int64_t nC, uint32_t nitems) {
    constexpr int NH = N / 2, NP = NH / WB, NTH = NH / 16;  // state half, passes, state tiles per wavefront
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Wide8Lds& sm = *reinterpret_cast<Wide8Lds*>(smem_raw);

    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int h = (int)(item % (uint32_t)H);
    const int64_t c = (item / (uint32_t)H) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)H * (uint32_t)nC);
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pt = w8 & 3, nh = w8 >> 2;  // p-tile and state half of this wavefront
    const float Dh = D ? D[h] : 0.0f;
    const int64_t t0 = c * Q;
    const int64_t t_end = t0 + Q < L ? t0 + Q : L;
    const int nsub = (int)((t_end - t0 + QS - 1) / QS);
    const int64_t nsubT = (L + QS - 1) / QS;
    float cs_prev = 0.0f, tot = 0.0f;

    // st[nt] holds S[p = 16 pt + l16][n = nh N/2 + 16 nt + 4 g4 + r]
    f32x4 st[NTH];
    {
        const float* S0 = start + ((b * nC + c) * H + h) * (int64_t)P * N + (int64_t)(16 * pt + l16) * N + nh * NH +
                          4 * g4;
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt) st[nt] = *reinterpret_cast<const f32x4*>(S0 + 16 * nt);
    }
    if (tid < 256) {
        sm.mb[(1 * 4 + 0) * 256 + tid] = static_cast<bf16>(0.0f);
        sm.mb[(3 * 4 + 2) * 256 + tid] = static_cast<bf16>(0.0f);
    }

    WideSrc src;
    src.x = x, src.B = B, src.C = C, src.ds = ds, src.b = b, src.L = L, src.H = H, src.G = G, src.N = N, src.h = h,
    src.g = g;
    src.dt0 = FWD ? ((b * H + h) * nsubT + c * (Q / QS)) * QS : ((b * H + h) * nC + c) * Q;
    const uint32_t xo = (uint32_t)(((tid >> 3) * (int64_t)H * P + (tid & 7) * 8) * 2);
    const uint32_t bo = (uint32_t)((((tid & 255) >> 4) * (int64_t)G * N + (tid >> 8) * (N / 2) + (tid & 15) * 8) * 2);
    Wide8Regs rg;
    wide8_load_x(rg, src, t0, 0, tid, xo);
    wide8_load_bc(rg, src, t0, 0, bo);
    const int64_t HP_ = (int64_t)H * P;
    const float* px = reinterpret_cast<const float*>(&sm.bs[0][0]);  // partial-output exchange area

    for (int sc = 0; sc < nsub; ++sc) {
        const int64_t tbase = t0 + (int64_t)sc * QS;
        const bool more = sc + 1 < nsub;
        __syncthreads();  // the previous sub-chunk's readers are done with the LDS tiles
        *reinterpret_cast<uint4*>(&sm.xs[(tid >> 3) * XS + (tid & 7) * 8]) = rg.x;
        if (tid < 64) wide_decay_store<FWD>(sm.lw, sm.dtw, sm.ww, sm.ec, sm.alpha, rg.dt, rg.cs, cs_prev, tot, tid);
        wide8_store_bc(sm, rg, tid);
        __syncthreads();
        if (more) wide8_load_x(rg, src, tbase + QS, sc + 1, tid, xo);
        if (NP > 1)
            wide8_load_bc(rg, src, tbase, 1, bo);
        else if (more)
            wide8_load_bc(rg, src, tbase + QS, 0, bo);

        Frag<bf16> xw[2];  // decay-scaled X^T fragments of p-tile pt
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            Frag<bf16> xf;
            xf.v = pack8(tr_read(sm.xs, 32 * ks + 4 * g4, 16 * pt, XS, l16),
                         tr_read(sm.xs, 32 * ks + 16 + 4 * g4, 16 * pt, XS, l16));
            const float* wv = &sm.ww[32 * ks + 4 * g4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                xw[ks].v[r] = static_cast<bf16>(static_cast<float>(xf.v[r]) * wv[r]);
                xw[ks].v[4 + r] = static_cast<bf16>(static_cast<float>(xf.v[4 + r]) * wv[16 + r]);
            }
        }
        const float alpha = sm.alpha[0];
        f32x4 acc[4], gacc[2];
#pragma unroll
        for (int it = 0; it < 4; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        gacc[0] = gacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int q = 0; q < NP; ++q) {
            if (q > 0) {
                __syncthreads();  // every wavefront is done with the previous pass's blocks
                wide8_store_bc(sm, rg, tid);
                __syncthreads();
                if (q + 1 < NP)
                    wide8_load_bc(rg, src, tbase, q + 1, bo);
                else if (more)
                    wide8_load_bc(rg, src, tbase + QS, 0, bo);
            }
            // C.B^T tiles w8 and w8 + 8 (of the ten in the lower triangle) over both blocks
#pragma unroll
            for (int o = 0; o < 2; ++o) {
                const int tt = w8 + 8 * o;
                if (tt < 10) {
                    const int it = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
                    const int jt = tt - it * (it + 1) / 2;
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
                        for (int ks = 0; ks < WB / 32; ++ks) {
                            Frag<bf16> a, bo;
                            frag_load8<bf16>(a, &sm.bs[hb][(16 * jt + l16) * WBS + 32 * ks + 8 * g4]);
                            frag_load8<bf16>(bo, &sm.cs[hb][(16 * it + l16) * WCS + 32 * ks + 8 * g4]);
                            mma(gacc[o], a, bo);
                        }
                    }
                }
            }
            // partial S C^T over this wavefront's block, from the state before the update
            const bf16* csb = sm.cs[nh];
#pragma unroll
            for (int ks = 0; ks < WB / 32; ++ks) {
                Frag<bf16> sa;
                sa.v = pack8(cvt4(st[q * (WB / 16) + 2 * ks]), cvt4(st[q * (WB / 16) + 2 * ks + 1]));
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const bf16* crow = &csb[(16 * it + l16) * WCS + 32 * ks];
                    Frag<bf16> bo;
                    bo.v = pack8(*reinterpret_cast<const bf16x4*>(crow + 4 * g4),
                                 *reinterpret_cast<const bf16x4*>(crow + 16 + 4 * g4));
                    mma(acc[it], sa, bo);
                }
            }
            // S <- 2^(l_63) S + B^T (w x) on this block's columns
#pragma unroll
            for (int nt = 0; nt < WB / 16; ++nt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) st[q * (WB / 16) + nt][r] *= alpha;
            }
            const bf16* bsb = sm.bs[nh];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int nt = 0; nt < WB / 16; ++nt) {
                    Frag<bf16> a;
                    a.v = pack8(tr_read(bsb, 32 * ks + 4 * g4, 16 * nt, WBS, l16),
                                tr_read(bsb, 32 * ks + 16 + 4 * g4, 16 * nt, WBS, l16));
                    mma(st[q * (WB / 16) + nt], a, xw[ks]);
                }
            }
        }
        __syncthreads();  // the blocks are free: their space takes the partial outputs

        // send the token tiles the other half finishes (half 0 finishes 0-1, half 1 finishes 2-3)
        float* pxw = reinterpret_cast<float*>(&sm.bs[0][0]);
        if (nh == 0) {
            *reinterpret_cast<f32x4*>(&pxw[((w8 * 2 + 0) * 64 + lane) * 4]) = acc[2];
            *reinterpret_cast<f32x4*>(&pxw[((w8 * 2 + 1) * 64 + lane) * 4]) = acc[3];
        } else {
            *reinterpret_cast<f32x4*>(&pxw[((w8 * 2 + 0) * 64 + lane) * 4]) = acc[0];
            *reinterpret_cast<f32x4*>(&pxw[((w8 * 2 + 1) * 64 + lane) * 4]) = acc[1];
        }
        // decayed C.B^T tiles -> LDS (D_h on the diagonal, so X^T M also yields D x)
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int tt = w8 + 8 * o;
            if (tt < 10) {
                const int it = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
                const int jt = tt - it * (it + 1) / 2;
                const int i = 16 * it + l16, j0 = 16 * jt + 4 * g4;
                f32x4 m;
                if (jt == it) {
                    const float li = sm.lw[i];
                    const f32x4 lj = *reinterpret_cast<const f32x4*>(&sm.lw[j0]);
                    const f32x4 dj = *reinterpret_cast<const f32x4*>(&sm.dtw[j0]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = gacc[o][r] * fast_exp2(fminf(li - lj[r], 0.0f)) * dj[r];
                        m[r] = (j0 + r <= i ? v : 0.0f) + (j0 + r == i ? Dh : 0.0f);
                    }
                } else {
                    const float er = sm.ec[i];
                    const f32x4 ej = *reinterpret_cast<const f32x4*>(&sm.ec[it * QS + j0]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[r] = gacc[o][r] * er * ej[r];
                }
                *reinterpret_cast<bf16x4*>(&sm.mb[((jt * 4 + it) * 64 + lane) * 4]) = cvt4(m);
            }
        }
        __syncthreads();

        // Y^T[p-tile pt] of the token tiles this half finishes
        const bool full = tbase + QS <= L;
        bf16* yb = y + ((b * L + tbase) * H + h) * (int64_t)P + 16 * pt + 4 * g4;
        const int partner = w8 ^ 4;  // same p-tile, other half
        if (nh == 0)
            wide8_finish<0>(acc, sm, px, partner, pt, lane, g4, l16, yb, HP_, full, L - tbase);
        else
            wide8_finish<2>(acc, sm, px, partner, pt, lane, g4, l16, yb, HP_, full, L - tbase);
    }
}

// ---------------------------------------------------------------------------
// chunk-local states (hi + lo split of the scaled operand, as in fused.hip): every token's contribution
// reaches the chunk's end through one weight 2^(l_end - l_j) dt_j, so the state is a plain sum over the
// chunk's tokens with no per-sub-chunk decay of the partial state; the sub-chunks are walked from the
// last, which makes each one's distance to the chunk's end known when its weights are formed
// ---------------------------------------------------------------------------
struct WideAggLds {
    bf16 xs[QS * XS];
    bf16 bs[QS * WBS];
    float ww[QS];  // 2^(l_end - l_j) dt_j
};

// x to LDS and the sub-chunk's weights (wavefront 0, lane = token).  FWD: the decay arrays restart at
// every sub-chunk and `after` holds the log2 decay from this sub-chunk's end to the chunk's end; tot
// accumulates the chunk's total.  Otherwise cs is cumulative over the chunk, cs_end its last value.
template <bool FWD>
__device__ __forceinline__ void wide_state_store_x(bf16* xs, float* ww, const WideRegs& rg, const WideAddr& a,
                                                   float& after, float cs_end, float& tot, int tid) {
#pragma unroll
    for (int k = 0; k < 2; ++k) *reinterpret_cast<uint4*>(xs + (a.xr + 32 * k) * XS + a.xc) = rg.x[k];
    if (tid < 64) {
        float e;  // log2 decay from this token to the chunk's end
        if (FWD) {
            const float last = __shfl(rg.cs, 63, 64);
            e = after + (last - rg.cs);
            after += last;
            tot += last;
        } else {
            e = cs_end - rg.cs;
        }
        ww[tid] = fast_exp2(e) * rg.dt;
    }
}

template <int N, bool FWD>
__global__ void __launch_bounds__(256, 2)
chunk_state_wide_kernel(const bf16* __restrict__ x, const bf16* __restrict__ B, DtSrc ds, float* __restrict__ states,
                        float* __restrict__ totals, int64_t L, int H, int G, int Q, int64_t nC, uint32_t nitems) {
    constexpr int NBLK = N / WB, NT = N / 16;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    WideAggLds& sm = *reinterpret_cast<WideAggLds*>(smem_raw);

    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int h = (int)(item % (uint32_t)H);
    const int64_t c = (item / (uint32_t)H) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)H * (uint32_t)nC);
    const int g = h / (H / G);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int64_t t0 = c * Q;
    const int64_t t_end = t0 + Q < L ? t0 + Q : L;
    const int nsub = (int)((t_end - t0 + QS - 1) / QS);
    const int64_t nsubT = (L + QS - 1) / QS;

    f32x4 st[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) st[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    WideSrc src;
    src.x = x, src.B = B, src.C = nullptr, src.ds = ds, src.b = b, src.L = L, src.H = H, src.G = G, src.N = N,
    src.h = h, src.g = g;
    src.dt0 = FWD ? ((b * H + h) * nsubT + c * (Q / QS)) * QS : ((b * H + h) * nC + c) * Q;
    float after = 0.0f, tot = 0.0f, cs_end = 0.0f;
    if (!FWD && tid < 64) cs_end = ds.cs[src.dt0 + (Q - 1)];
    WideAddr ad;
    wide_addr(ad, src, tid);
    WideRegs rg;
    {
        const int64_t tl = t0 + (int64_t)(nsub - 1) * QS;
        wide_load_x(rg, ad, src, tl, nsub - 1, tid);
        wide_load_bc<false>(rg, ad, src, tl, 0);
    }

    for (int sc = nsub - 1; sc >= 0; --sc) {
        const int64_t tbase = t0 + (int64_t)sc * QS;
        const bool more = sc > 0;
        __syncthreads();
        wide_state_store_x<FWD>(sm.xs, sm.ww, rg, ad, after, cs_end, tot, tid);
        wide_store_bc<false>(sm.bs, nullptr, rg, ad);
        __syncthreads();
        if (more) wide_load_x(rg, ad, src, tbase - QS, sc - 1, tid);
        if (NBLK > 1)
            wide_load_bc<false>(rg, ad, src, tbase, 1);
        else if (more)
            wide_load_bc<false>(rg, ad, src, tbase - QS, 0);

        Frag<bf16> xh[2], xl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 lo4 = tr_read(sm.xs, 32 * ks + 4 * g4, 16 * w, XS, l16);
            const bf16x4 hi4 = tr_read(sm.xs, 32 * ks + 16 + 4 * g4, 16 * w, XS, l16);
            const float* wv = &sm.ww[32 * ks + 4 * g4];
            // four values at a time; the hi part is read back from its packed pair
            const f32x4 w0 = {wv[0], wv[1], wv[2], wv[3]}, w1 = {wv[16], wv[17], wv[18], wv[19]};
            const f32x4 v0 = __builtin_convertvector(lo4, f32x4) * w0;
            const f32x4 v1 = __builtin_convertvector(hi4, f32x4) * w1;
            const bf16x4 h0 = __builtin_convertvector(v0, bf16x4), h1 = __builtin_convertvector(v1, bf16x4);
            xh[ks].v = pack8(h0, h1);
            xl[ks].v = pack8(__builtin_convertvector(v0 - bf16x4_to_f32(h0), bf16x4),
                             __builtin_convertvector(v1 - bf16x4_to_f32(h1), bf16x4));
        }
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb) {
            if (nb > 0) {
                __syncthreads();
                wide_store_bc<false>(sm.bs, nullptr, rg, ad);
                __syncthreads();
                if (nb + 1 < NBLK)
                    wide_load_bc<false>(rg, ad, src, tbase, nb + 1);
                else if (more)
                    wide_load_bc<false>(rg, ad, src, tbase - QS, 0);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int nt = 0; nt < WB / 16; ++nt) {
                    Frag<bf16> a;
                    a.v = pack8(tr_read(sm.bs, 32 * ks + 4 * g4, 16 * nt, WBS, l16),
                                tr_read(sm.bs, 32 * ks + 16 + 4 * g4, 16 * nt, WBS, l16));
                    mma(st[nb * (WB / 16) + nt], a, xh[ks]);
                    mma(st[nb * (WB / 16) + nt], a, xl[ks]);
                }
            }
        }
    }
    // a ragged last chunk ends at position Q-1 all the same: its padded tokens have dt = 0 and decay 1
    float* out = states + ((b * nC + c) * H + h) * (int64_t)P * N + (int64_t)(16 * w + l16) * N + 4 * g4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(out + 16 * nt) = st[nt];
    if (FWD && tid == 0) totals[(b * H + h) * nC + c] = tot;
}

// ---------------------------------------------------------------------------
// the same chunk-local states on 32 x 32 x 16 MFMAs.  The state is held transposed, S^T (n x p), in 32 x 32
// accumulator tiles: wavefront w owns p-tile w % 2 (32 rows of p) and state half w / 2 (N/2 columns of n),
// N/64 tiles.  Lane l of a 32 x 32 x 16 product holds operand row (A) or column (B) l % 32 and K positions
// 8 (l / 32) .. + 7; accumulator slot i of lane l is row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
// The A operand B^T (n x tokens) and the B operand w x (tokens x p) come from transpose reads of the
// natural-layout tiles with the same token order (16-lane group g reads tokens 16 ks + 8 (g / 2) ..), so
// one operand fetch serves twice the products of the 16 x 16 x 32 form and every B column is read by two
// wavefronts instead of four.  Each pass stages one 128-column block per half.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void mma32(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}

struct Wide32Lds {
    bf16 xs[QS * XS];
    bf16 bs[2][QS * WBS];  // this pass's block of each half
    uint4 xf[4][4][2][64];  // per wavefront, K step, hi / lo: the scaled operand in fragment order
    float ww[QS];           // 2^(l_end - l_j) dt_j
};

struct Wide32Regs {
    uint4 x[2];
    uint4 b[8];  // the pass's two blocks: half tid / 128, rows (tid % 128) / 16 + 8 k, columns 8 (tid % 16)
    float dt, cs;
};

template <int N, bool FWD>
__global__ void __launch_bounds__(256, 2)
chunk_state_wide32_kernel(const bf16* __restrict__ x, const bf16* __restrict__ B, DtSrc ds, float* __restrict__ states,
                          float* __restrict__ totals, int64_t L, int H, int G, int Q, int64_t nC, uint32_t nitems) {
    constexpr int NH = N / 2, NPASS = NH / WB, NTW = NH / 32;  // state half, passes, 32-wide tiles per wavefront
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Wide32Lds& sm = *reinterpret_cast<Wide32Lds*>(smem_raw);

    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int h = (int)(item % (uint32_t)H);
    const int64_t c = (item / (uint32_t)H) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)H * (uint32_t)nC);
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pt = w & 1, nh = w >> 1;  // p-tile and state half of this wavefront
    const int64_t t0 = c * Q;
    const int64_t t_end = t0 + Q < L ? t0 + Q : L;
    const int nsub = (int)((t_end - t0 + QS - 1) / QS);
    const int64_t nsubT = (L + QS - 1) / QS;

    f32x16 st[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[t][i] = 0.0f;

    WideSrc src;
    src.x = x, src.B = B, src.C = nullptr, src.ds = ds, src.b = b, src.L = L, src.H = H, src.G = G, src.N = N,
    src.h = h, src.g = g;
    src.dt0 = FWD ? ((b * H + h) * nsubT + c * (Q / QS)) * QS : ((b * H + h) * nC + c) * Q;
    float after = 0.0f, tot = 0.0f, cs_end = 0.0f;
    if (!FWD && tid < 64) cs_end = ds.cs[src.dt0 + (Q - 1)];
    WideAddr ad;
    wide_addr(ad, src, tid);
    // the B pieces of this thread: half bh, rows br + 8 k, columns 8 (tid % 16) of the half's block q
    const int bh = tid >> 7, br = (tid & 127) >> 4, bc = (tid & 15) * 8;
    const int64_t GN = (int64_t)G * N;
    const uint32_t bo = (uint32_t)((br * GN + bh * NH + bc) * 2);
    auto load_b = [&](Wide32Regs& rg, int64_t tb, int q) {
        const auto rb = tile_rsrc(B + ((b * L + tb) * G + g) * (int64_t)N, GN, L - tb, N);
#pragma unroll
        for (int k = 0; k < 8; ++k) rg.b[k] = ldbuf(rb, bo + (uint32_t)((8 * k * GN + WB * q) * 2));
    };
    auto load_x = [&](Wide32Regs& rg, int64_t tb, int sub) {
        const int64_t HP_ = (int64_t)H * P;
        const auto r = tile_rsrc(x + ((b * L + tb) * H + h) * (int64_t)P, HP_, L - tb, P);
#pragma unroll
        for (int k = 0; k < 2; ++k) rg.x[k] = ldbuf(r, ad.xo + (uint32_t)(32 * k * HP_ * 2));
        if (tid < 64) {
            rg.dt = ds.dt_t[src.dt0 + (int64_t)QS * sub + tid];
            rg.cs = ds.cs[src.dt0 + (int64_t)QS * sub + tid];
        }
    };
    auto store_b = [&](const Wide32Regs& rg) {
#pragma unroll
        for (int k = 0; k < 8; ++k) *reinterpret_cast<uint4*>(&sm.bs[bh][(br + 8 * k) * WBS + bc]) = rg.b[k];
    };
    Wide32Regs rg;
    {
        const int64_t tl = t0 + (int64_t)(nsub - 1) * QS;
        load_x(rg, tl, nsub - 1);
        load_b(rg, tl, 0);
    }
    // transpose-read coordinates of this lane: token rows 16 ks + 8 (grp / 2) (+ 4), columns 16 (grp % 2) ..
    const int krow = 8 * (grp >> 1), kcol = 16 * (grp & 1);

    for (int sc = nsub - 1; sc >= 0; --sc) {
        const int64_t tbase = t0 + (int64_t)sc * QS;
        const bool more = sc > 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 2; ++k) *reinterpret_cast<uint4*>(sm.xs + (ad.xr + 32 * k) * XS + ad.xc) = rg.x[k];
        if (tid < 64) {
            float e;  // log2 decay from this token to the chunk's end
            if (FWD) {
                const float last = __shfl(rg.cs, 63, 64);
                e = after + (last - rg.cs);
                after += last;
                tot += last;
            } else {
                e = cs_end - rg.cs;
            }
            sm.ww[tid] = fast_exp2(e) * rg.dt;
        }
        store_b(rg);
        __syncthreads();
        if (more) load_x(rg, tbase - QS, sc - 1);
        if (NPASS > 1)
            load_b(rg, tbase, 1);
        else if (more)
            load_b(rg, tbase - QS, 0);

        // the scaled operand w x of p-tile pt, hi + lo, for the four 16-token K steps, parked in this
        // wavefront's LDS slot in fragment order (fewer live registers through the passes)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x4 v0 = tr_read(sm.xs, 16 * ks + krow, 32 * pt + kcol, XS, l16);
            const bf16x4 v1 = tr_read(sm.xs, 16 * ks + krow + 4, 32 * pt + kcol, XS, l16);
            const float* wv = &sm.ww[16 * ks + krow];
            Frag<bf16> xh, xl;
            // four values at a time; the hi part is read back from its packed pair
            const f32x4 w0 = {wv[0], wv[1], wv[2], wv[3]}, w1 = {wv[4], wv[5], wv[6], wv[7]};
            const f32x4 a0 = __builtin_convertvector(v0, f32x4) * w0;
            const f32x4 a1 = __builtin_convertvector(v1, f32x4) * w1;
            const bf16x4 h0 = __builtin_convertvector(a0, bf16x4), h1 = __builtin_convertvector(a1, bf16x4);
            xh.v = pack8(h0, h1);
            xl.v = pack8(__builtin_convertvector(a0 - bf16x4_to_f32(h0), bf16x4),
                         __builtin_convertvector(a1 - bf16x4_to_f32(h1), bf16x4));
            *reinterpret_cast<bf16x8*>(&sm.xf[w][ks][0][lane]) = xh.v;
            *reinterpret_cast<bf16x8*>(&sm.xf[w][ks][1][lane]) = xl.v;
        }
#pragma unroll
        for (int q = 0; q < NPASS; ++q) {
            if (q > 0) {
                __syncthreads();
                store_b(rg);
                __syncthreads();
                if (q + 1 < NPASS)
                    load_b(rg, tbase, q + 1);
                else if (more)
                    load_b(rg, tbase - QS, 0);
            }
            const bf16* bsb = sm.bs[nh];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Frag<bf16> xh, xl;
                xh.v = *reinterpret_cast<const bf16x8*>(&sm.xf[w][ks][0][lane]);
                xl.v = *reinterpret_cast<const bf16x8*>(&sm.xf[w][ks][1][lane]);
#pragma unroll
                for (int t = 0; t < WB / 32; ++t) {
                    Frag<bf16> a;
                    a.v = pack8(tr_read(bsb, 16 * ks + krow, 32 * t + kcol, WBS, l16),
                                tr_read(bsb, 16 * ks + krow + 4, 32 * t + kcol, WBS, l16));
                    mma32(st[q * (WB / 32) + t], a, xh);
                    mma32(st[q * (WB / 32) + t], a, xl);
                }
            }
        }
    }
    // a ragged last chunk ends at position Q-1 all the same: its padded tokens have dt = 0 and decay 1
    float* out = states + ((b * nC + c) * H + h) * (int64_t)P * N + (int64_t)(32 * pt + (lane & 31)) * N + nh * NH +
                 4 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 v = {st[t][4 * i4], st[t][4 * i4 + 1], st[t][4 * i4 + 2], st[t][4 * i4 + 3]};
            *reinterpret_cast<f32x4*>(out + 32 * t + 8 * i4) = v;
        }
    }
    if (FWD && tid == 0) totals[(b * H + h) * nC + c] = tot;
}

template <int N, bool FWD>
hipError_t launch_state_wide(const Shape& s, const bf16* x, const bf16* B, const DtSrc& ds, float* states,
                             float* totals, hipStream_t st) {
    const uint32_t nitems = (uint32_t)(s.b * s.nC * s.H);
    if (nitems == 0) return hipSuccess;
    // dstate 512: the 32 x 32 x 16 form (64K-token forward 1.09-1.10 against 1.11-1.12 ms on two boxes, 4.18
    // against 4.21 ms at 256K: half the MFMA issues and operand reads, little time, so the kernel is bound by
    // neither).  dstate 256 keeps the 16 x 16 x 32 form: the 32 x 32 one's LDS (80 KB) halves its residency
    // and measured 0.59 against 0.57 ms (2.21 against 2.06 ms at 256K).
    if constexpr (N >= 512) {
        const size_t lds = sizeof(Wide32Lds);
        hipError_t e = hipFuncSetAttribute((const void*)chunk_state_wide32_kernel<N, FWD>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((chunk_state_wide32_kernel<N, FWD>), dim3(nitems), dim3(256), lds, st, x, B, ds, states,
                           totals, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems);
        return hipGetLastError();
    }
    const size_t lds = sizeof(WideAggLds);
    hipError_t e = hipFuncSetAttribute((const void*)chunk_state_wide_kernel<N, FWD>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_state_wide_kernel<N, FWD>), dim3(nitems), dim3(256), lds, st, x, B, ds, states, totals,
                       s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems);
    return hipGetLastError();
}

template <int N, bool FWD>
hipError_t launch_scan_wide(const Shape& s, const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                            const float* start, const float* D, bf16* y, hipStream_t st) {
    const uint32_t nitems = (uint32_t)(s.b * s.nC * s.H);
    if (nitems == 0) return hipSuccess;
    // dstate 512: the split-state kernel (two wavefronts per SIMD instead of one; measured 5.80 against
    // 6.79 ms for the 256K-token forward).  dstate 256 keeps the four-wavefront kernel, which already
    // runs two workgroups per CU (the split one measured 3.04 against 2.65 ms there).
    if constexpr (N >= 512) {
        const size_t lds8 = sizeof(Wide8Lds);
        hipError_t e = hipFuncSetAttribute((const void*)chunk_scan_wide8_kernel<N, FWD>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds8);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((chunk_scan_wide8_kernel<N, FWD>), dim3(nitems), dim3(512), lds8, st, x, B, C, ds, start,
                           D, y, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems);
        return hipGetLastError();
    }
    const size_t lds = sizeof(WideScanLds);
    hipError_t e = hipFuncSetAttribute((const void*)chunk_scan_wide_kernel<N, FWD>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_scan_wide_kernel<N, FWD>), dim3(nitems), dim3(256), lds, st, x, B, C, ds, start, D, y,
                       s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems);
    return hipGetLastError();
}

template <bool FWD>
hipError_t state_wide(const Shape& s, const bf16* x, const bf16* B, const DtSrc& ds, float* states, float* totals,
                      hipStream_t st) {
    return s.N == 512 ? launch_state_wide<512, FWD>(s, x, B, ds, states, totals, st)
                      : launch_state_wide<256, FWD>(s, x, B, ds, states, totals, st);
}

template <bool FWD>
hipError_t scan_wide(const Shape& s, const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                     const float* start, const float* D, bf16* y, hipStream_t st) {
    return s.N == 512 ? launch_scan_wide<512, FWD>(s, x, B, C, ds, start, D, y, st)
                      : launch_scan_wide<256, FWD>(s, x, B, C, ds, start, D, y, st);
}

template hipError_t state_wide<false>(const Shape&, const bf16*, const bf16*, const DtSrc&, float*, float*,
                                      hipStream_t);
template hipError_t state_wide<true>(const Shape&, const bf16*, const bf16*, const DtSrc&, float*, float*,
                                     hipStream_t);
template hipError_t scan_wide<false>(const Shape&, const bf16*, const bf16*, const bf16*, const DtSrc&, const float*,
                                     const float*, bf16*, hipStream_t);
template hipError_t scan_wide<true>(const Shape&, const bf16*, const bf16*, const bf16*, const DtSrc&, const float*,
                                    const float*, bf16*, hipStream_t);

}  // namespace fz
}  // namespace ssd
