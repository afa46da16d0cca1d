// fused.hip -- fast chunk-state and chunk-scan kernels for bf16 inputs with
// headdim 64 and dstate 64 or 128, for any chunk size Q that is a multiple of 64.
//
// They compute exactly the staged calls of the cuTile Mamba-2 page (devotd.net,
// section 2): the chunk-local states, and the chunk output from the chunk-start
// state.  Inside a chunk they walk 64-token sub-chunks, which is the same
// recurrence regrouped once more ("3.3 Hardware-Aware algorithms ...", section
// 4.1, associativity):
//
//   chunk_state_fast_kernel  per (b, chunk, head pair): S = sum_j B_j (outer) (w_j x_j)
//                            over the chunk's tokens with w_j = 2^(l_end - l_j) dt_j,
//                            sub-chunks walked from the last, with the scaled operand
//                            split into hi + lo bf16 parts (fp32-level state).
//   chunk_scan_fast_kernel   per (b, chunk, head pair): carry the fp32 state in
//                            registers from the chunk-start state; per sub-chunk
//                              y  = 2^(l_i) C_i . S + sum_{j<=i} (C_i . B_j) 2^(l_i-l_j) dt_j x_j + D x_i
//                              S <- 2^(l_63) S + sum_j 2^(l_63-l_j) dt_j B_j (outer) x_j
//                            with l relative to the sub-chunk start.  Only y is written.
//
// With a large chunk (a few thousand tokens) the per-chunk states are few, so
// the forward's state traffic through HBM stays small while every kernel still
// has thousands of independent work items.
//
// Layout choices (gfx950):
//   * x, B and C sub-chunks sit in LDS in their natural row-major layout.
//     Operands whose contraction runs over tokens (X^T, B^T) are fetched with the
//     LDS transpose read (ds_read_b64_tr_b16: a 16-lane group reads a 4 x 16
//     block and each lane receives one column); nothing is transposed in
//     registers.
//   * Row strides make the fragment reads bank-conflict-free: x rows of 80 bf16
//     and B rows of N+16 bf16 (transpose reads of 8 rows land in 8 distinct
//     8-bank groups), C rows of N+8 bf16 (row reads of 16 rows).
//   * The output is computed transposed, Y^T = S C^T + X^T M, so the carried
//     state feeds the MFMA straight from its accumulator registers, and the
//     decayed C.B^T tiles are stored in LDS in fragment order.
//   * Two heads share a workgroup: the B and C tiles, the C.B^T tiles and the C
//     and B^T fragments are loaded once for both heads.
//   * The decay is formed in fp32 with exp2; the upper triangle is selected to
//     zero before use (static masking).
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ssd {
namespace fz {

// ---------------------------------------------------------------------------
// chunk staging shared by both kernels: x (HPW heads), B, C (optional), dt
// ---------------------------------------------------------------------------
template <int N, int HPW, bool WITH_C>
struct ChunkRegs {
    uint4 x[2 * HPW];
    uint4 b[N / 32];
    uint4 c[WITH_C ? N / 32 : 1];
    float dt;   // dt_t of token (tid & 63) of head (tid >> 6), threads < 64 * HPW
    float cs;   // chunk cumulative log2 decay of that token
    float rs;   // its output row scale (reversed walk with a row scale only)
};

// Per-thread staging offsets within one sub-chunk tile, in bytes from the tile's first element (32-bit: a
// tile spans 64 tokens).  Chunk k of a thread is chunk (tid + 256 k) of the tile: x chunk k covers head
// k / 2, rows (tid / 8) + 32 (k % 2); B / C chunk k covers row tid / (N / 8) + k * RPI.  The tiles are
// read through wavefront-uniform buffer resources, so each load is a resource plus this offset plus a
// uniform constant.
template <int N, int HPW>
struct ChunkAddr {
    uint32_t xo, bo, dto;  // byte offsets of this thread's first x and B/C piece; dt/cs element
    int xl, bl, cl;        // LDS element offsets of the first x / B / C chunk
};

template <int N>
struct BRows {
    static constexpr int RPI = 256 / (N / 8);  // B rows covered by one pass of 256 threads
};


// wavefront-uniform bases of one sub-chunk's tiles
struct TileBase {
    const bf16 *x, *b, *c;
    const float *dt, *cs;
    const bf16* rdt;  // raw dt (DtSrc::raw): the sub-chunk's first row, this workgroup's first head
    int64_t rows;     // rows of the tile inside the inputs, from the resource's start
};

// hx: heads of the x rows; dt_head: distance between consecutive heads in the dt/cs arrays.
// REV: the tile's rows run backwards from its last input row (the resource starts at the lowest one), so
// tile row r sits 63 - r rows above the resource's start; the later pieces of a thread step downwards.
// RAW: dt_head is the row length of the raw dt (its heads), and a thread's dt element is token r, head hh.
template <int N, int HPW, bool REV = false, bool RAW = false>
__device__ __forceinline__ void chunk_addr(ChunkAddr<N, HPW>& a, int hx, int G, int64_t dt_head, int tid) {
    constexpr int BS = Strides<N>::BS, CS = Strides<N>::CS;
    const int xr = tid >> 3, xc = (tid & 7) * 8;
    a.xo = (uint32_t)((REV ? QS - 1 - xr : xr) * hx * P + xc) * 2u;
    a.xl = xr * XS + xc;
    const int br = tid / (N / 8), bc = (tid % (N / 8)) * 8;
    a.bo = (uint32_t)((REV ? QS - 1 - br : br) * G * N + bc) * 2u;
    a.bl = br * BS + bc;
    a.cl = br * CS + bc;
    const int hh = tid >> 6, r = tid & 63;
    a.dto = RAW ? (uint32_t)(r * dt_head + (hh < HPW ? hh : 0)) : (uint32_t)((hh < HPW ? hh : 0) * dt_head + r);
}

// The tiles of the sub-chunk starting at token tbase of batch row b (x heads xh0.. of hx per row,
// group g); dt0 / cs0 point at this chunk's first position of the workgroup's first head and sub is the
// sub-chunk index.  REV: the inputs hold Lin rows per batch row in forward time, token t is input row
// L - 1 - t, so the tile covers input rows L - 64 - tbase (its last token, the resource's start) up to
// L - 1 - tbase, of which those below Lin exist (L a multiple of 64).
template <bool WITH_C, bool REV = false, bool RAW = false>
__device__ __forceinline__ TileBase tile_base(const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                                              int64_t dt0, int64_t b, int64_t L, int hx, int G, int N, int xh0, int g,
                                              int64_t tbase, int sub, int64_t Lin = 0) {
    TileBase t;
    const int64_t r0 = REV ? b * Lin + (L - QS - tbase) : b * L + tbase;  // the resource's first row
    t.x = x + (r0 * hx + xh0) * (int64_t)P;
    t.b = B + (r0 * G + g) * (int64_t)N;
    t.c = WITH_C ? C + (r0 * G + g) * (int64_t)N : nullptr;
    t.rows = REV ? Lin - (L - QS - tbase) : L - tbase;
    if constexpr (RAW) {  // dt0: the raw element of token 0 of this batch row and the workgroup's first head
        t.rdt = ds.raw + dt0 + tbase * (int64_t)ds.H;
        t.dt = t.cs = nullptr;
    } else {
        t.rdt = nullptr;
        t.dt = ds.dt_t + dt0 + (int64_t)QS * sub;
        t.cs = ds.cs + dt0 + (int64_t)QS * sub;
    }
    return t;
}

// Load one sub-chunk into registers; rows past the inputs' end read as zero (t.rows from the resource's
// start).  REV (offsets from chunk_addr<REV>): a thread's later pieces lie 32 or RPI rows lower.
// RAW: rg.dt is the raw step and rg.cs flags a token inside the sequence.
template <int N, int HPW, bool WITH_C, bool REV = false, bool RAW = false>
__device__ __forceinline__ void chunk_load(ChunkRegs<N, HPW, WITH_C>& rg, const ChunkAddr<N, HPW>& a,
                                           const TileBase& t, int hx, int G, int tid) {
    constexpr int RPI = BRows<N>::RPI;
    const uint32_t HP_ = (uint32_t)(hx * P), GN = (uint32_t)(G * N);
    if (tid < 64 * HPW) {
        if (RAW) {
            const bool in = (tid & 63) < t.rows;
            rg.dt = in ? to_f32(t.rdt[a.dto]) : 0.0f;
            rg.cs = in ? 1.0f : 0.0f;
        } else {  // dt_t and cs cover every position of the chunk (zero-padded past L)
            rg.dt = t.dt[a.dto];
            rg.cs = t.cs[a.dto];
        }
    }
    const auto rx = tile_rsrc(t.x, HP_, t.rows, HPW * P);
    const auto rb = tile_rsrc(t.b, GN, t.rows, N);
#pragma unroll
    for (int k = 0; k < 2 * HPW; ++k)
        rg.x[k] = ldbuf(rx, (REV ? a.xo - (k & 1) * 32 * HP_ * 2u : a.xo + (k & 1) * 32 * HP_ * 2u) + (k >> 1) * P * 2u);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) rg.b[k] = ldbuf(rb, REV ? a.bo - k * RPI * GN * 2u : a.bo + k * RPI * GN * 2u);
    if (WITH_C) {
        const auto rc = tile_rsrc(t.c, GN, t.rows, N);
#pragma unroll
        for (int k = 0; k < N / 32; ++k) rg.c[k] = ldbuf(rc, REV ? a.bo - k * RPI * GN * 2u : a.bo + k * RPI * GN * 2u);
    }
}

// registers -> LDS, and the in-chunk cumulative decay (one wavefront per head)
// cs_prev: the chunk cumulative decay before this sub-chunk (0 for the first),
// held by wavefront hh for head hh and advanced here.
// With FWD the decay arrays already restart at the sub-chunk.  tot accumulates
// the sub-chunk totals (the chunk's total decay).
//
// ec (optional, [hh][4][64]): for the off-diagonal 16 x 16 tiles of the in-chunk
// matrix, 2^(l_i - l_j) dt_j = ec[0][i] * ec[it][j] with row-block start r = 16 it:
//   ec[0][i]  = 2^(l_i - l_(16 (i / 16)))      (<= 1: i at or after its block start)
//   ec[it][j] = 2^(l_(16 it) - l_j) dt_j       (<= dt_j for j < 16 it, the only ones used)
// so those tiles need no exponential; the diagonal tiles form 2^(l_i - l_j) directly.
// RAW (with FWD): rg holds the raw step (chunk_load<RAW>); the front-end fe with A[h] = ah gives the input
// and decay steps, and a wavefront scan of the decay steps the sub-chunk's cumulative decay.
template <int N, int HPW, bool WITH_C, bool FWD, bool RAW = false>
__device__ __forceinline__ void chunk_store(bf16* xs, bf16* bsm, bf16* csm, float* lw, float* dtw, float* ww,
                                            float* ec, float* alpha, const ChunkRegs<N, HPW, WITH_C>& rg,
                                            const ChunkAddr<N, HPW>& a, float& cs_prev, float& tot, int tid,
                                            const DtFront* fe = nullptr, int h = 0, float ah = 0.0f) {
    constexpr int RPI = BRows<N>::RPI, BS = Strides<N>::BS, CS = Strides<N>::CS;
#pragma unroll
    for (int k = 0; k < 2 * HPW; ++k)
        *reinterpret_cast<uint4*>(xs + a.xl + (k >> 1) * QS * XS + (k & 1) * 32 * XS) = rg.x[k];
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        *reinterpret_cast<uint4*>(bsm + a.bl + k * RPI * BS) = rg.b[k];
        if (WITH_C) *reinterpret_cast<uint4*>(csm + a.cl + k * RPI * CS) = rg.c[k];
    }
    if (tid < 64 * HPW) {
        const int hh = tid >> 6, lane = tid & 63;
        float d = rg.dt;
        float incl;  // cumulative log2 decay inside the sub-chunk
        if (RAW) {
            float dec = 0.0f, inp = 0.0f;  // zero past the sequence end
            if (rg.cs != 0.0f) dt_front(*fe, h, ah, rg.dt, dec, inp);
            d = inp;
            incl = wave_incl_scan(dec * ah) * kLog2e;
        } else if (FWD) {
            incl = rg.cs;
        } else {
            incl = rg.cs - cs_prev;
            cs_prev = lane_read(rg.cs, 63);
        }
        const float last = lane_read(incl, 63);
        tot += last;
        lw[hh * QS + lane] = incl;
        dtw[hh * QS + lane] = d;
        ww[hh * QS + lane] = fast_exp2(last - incl) * d;
        if (ec) {
            ec[(hh * 4) * QS + lane] = fast_exp2(incl - row_first(incl, lane));
#pragma unroll
            for (int it = 1; it < 4; ++it)
                ec[(hh * 4 + it) * QS + lane] = fast_exp2(fminf(lane_read(incl, 16 * it) - incl, 0.0f)) * d;
        }
        if (lane == 0) alpha[hh] = fast_exp2(last);
    }
}

// ---------------------------------------------------------------------------
// fused output kernel
// ---------------------------------------------------------------------------
template <int N, int HPW>
struct ScanLds {
    bf16 xs[HPW * QS * XS];         // x [hh][j][p]
    bf16 bs[QS * Strides<N>::BS];   // B [j][n]
    bf16 cs[QS * Strides<N>::CS];   // C [i][n]
    bf16 mb[HPW * 16 * 256];        // decayed C.B^T tiles, fragment order [hh][jt*4+it][lane][4]
    float lw[HPW * QS];             // in-chunk cumulative log2 decay
    float dtw[HPW * QS];            // dt
    float ww[HPW * QS];             // 2^(l_63 - l_j) dt_j
    float ec[HPW * 4 * QS];         // separable decay factors of the off-diagonal tiles (chunk_store)
    float rs[HPW * QS];             // output row scales (reversed walk with a row scale)
    float alpha[4];                 // 2^(l_63) per head
};


// FWD: sub-chunk-local decay arrays (subchunk_decay_kernel), as the forward reads them.
// REV (with FWD): the inputs are walked backwards and the output written forwards (XMap::rows); TAP
// (with FWD): the carried state is stored every XMap::tapq positions, with a hi/lo state update; TTR
// (with TAP): it is a transposed scan's state, stored back in its heads' layout (XMap::tap_tr).  RAW (with
// FWD, forwards, no taps): the decays come from the raw dt (DtSrc::raw), formed per sub-chunk in registers.
template <int N, int HPW, bool FWD, bool REV = false, bool TAP = false, bool TTR = false, bool RAW = false>
__global__ void __launch_bounds__(256, 2)
chunk_scan_fast_kernel(const bf16* __restrict__ x, const bf16* __restrict__ B, const bf16* __restrict__ C,
                       DtSrc ds, const float* __restrict__ start, const float* __restrict__ D, bf16* __restrict__ y, int64_t L,
                       int H, int G, int Q, int64_t nC, uint32_t nitems, XMap xm) {
    constexpr int NT = N / 16, NK = N / 32;
    constexpr int BS = Strides<N>::BS, CS = Strides<N>::CS;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ScanLds<N, HPW>& sm = *reinterpret_cast<ScanLds<N, HPW>*>(smem_raw);

    const int HP = H / HPW;
    const uint32_t item = xcd_remap_rev(blockIdx.x, nitems);
    const int hp = (int)(item % (uint32_t)HP);
    const int64_t c = (item / (uint32_t)HP) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)HP * (uint32_t)nC);
    const int h0 = hp * HPW;
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index, in a scalar register
    static_assert(!RAW || (FWD && !REV && !TAP), "raw decays: the forward's scan only");
    float Dh[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) Dh[hh] = D ? D[h0 + hh] : 0.0f;
    const int64_t t0 = c * Q;
    const int64_t t_end = t0 + Q < L ? t0 + Q : L;
    const int nsub = (int)((t_end - t0 + QS - 1) / QS);
    float cs_prev = 0.0f, tot = 0.0f;

    // carried state per head, transposed: st[hh][nt] holds S[p = 16w + l16][n = 16nt + 4g4 + r]
    f32x4 st[HPW][NT];
    if (REV && xm.start_tr) {  // a transposed scan's states: element (p, n) of head h at half-head n / 64, row n % 64
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int n = 16 * nt + 4 * g4;
                const float* S0 = start + (((b * nC + c) * H + h0 + hh) * (N / 64) + n / 64) * (int64_t)64 * P +
                                  (int64_t)(n % 64) * P + 16 * w + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) st[hh][nt][r] = S0[r * P];
            }
        }
    } else {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            const float* S0 =
                start + ((b * nC + c) * H + h0 + hh) * (int64_t)P * N + (int64_t)(16 * w + l16) * N + 4 * g4;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) st[hh][nt] = *reinterpret_cast<const f32x4*>(S0 + 16 * nt);
        }
    }
    // tiles above the diagonal that pair with a diagonal tile in a 32-wide K step stay zero
    for (int e = tid; e < HPW * 256; e += 256) {
        const int hh = e >> 8, q = e & 255;
        sm.mb[(hh * 16 + 1 * 4 + 0) * 256 + q] = static_cast<bf16>(0.0f);
        sm.mb[(hh * 16 + 3 * 4 + 2) * 256 + q] = static_cast<bf16>(0.0f);
    }

    const int64_t nsubT = (L + QS - 1) / QS;
    // dt/cs distance between heads (RAW: the raw dt's row length) and this chunk's first element
    const int64_t dt_head = RAW ? (int64_t)ds.H : FWD ? nsubT * QS : nC * Q;
    const int64_t dt0 = RAW   ? b * L * ds.H + h0
                        : FWD ? ((b * H + h0) * nsubT + c * (Q / QS)) * QS
                              : ((b * H + h0) * nC + c) * Q;
    const float ah = RAW && tid < 64 * HPW ? ds.A[h0 + (tid >> 6)] : 0.0f;  // A of this thread's head
    const int xh0 = h0 / xm.div * xm.mul;  // the x heads of this head pair
    ChunkAddr<N, HPW> ad;
    chunk_addr<N, HPW, REV, RAW>(ad, xm.hx, G, dt_head, tid);
    ChunkRegs<N, HPW, true> rg;
    chunk_load<N, HPW, true, REV, RAW>(rg, ad, tile_base<true, REV, RAW>(x, B, C, ds, dt0, b, L, xm.hx, G, N, xh0, g, t0, 0, xm.rows),
                                  xm.hx, G, tid);
    // reversed walk: the output row scale of token (tid & 63) of head (tid >> 6), at input row L - 1 - t
    const bf16* rsrc = REV ? static_cast<const bf16*>(xm.rowscale) : nullptr;
    auto load_rs = [&](int64_t tb) {
        if (REV && rsrc && tid < 64 * HPW) {
            const int64_t f = L - 1 - (tb + (tid & 63));
            rg.rs = f < xm.rows ? static_cast<float>(rsrc[(b * xm.rows + f) * H + h0 + (tid >> 6)]) : 0.0f;
        }
    };
    load_rs(t0);
    // this thread's output element offset within a sub-chunk's y tile (row l16, columns 16w + 4g4 ..)
    const uint32_t yo = (uint32_t)(l16 * H * P + 16 * w + 4 * g4);

    for (int sc = 0; sc < nsub; ++sc) {
        const int64_t tbase = t0 + (int64_t)sc * QS;
        if (TAP && tbase % xm.tapq == 0) {  // the state entering this position
            const int64_t tk = b * ((L + xm.tapq - 1) / xm.tapq) + tbase / xm.tapq;
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                if constexpr (TTR) {  // a transposed scan's state, back in its head's (dstate x headdim) layout
                    // (dword stores, 64 contiguous bytes per 16 lanes; a quad-lane transpose to 16-byte stores
                    // measured slower)
                    const int nh = xm.tap_tr, h2 = h0 + hh;
                    float* out = xm.tap + (tk * (H / nh) + h2 / nh) * (int64_t)N * (64 * nh) + 64 * (h2 % nh) +
                                 16 * w + l16;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) out[(int64_t)(16 * nt + 4 * g4 + r) * (64 * nh)] = st[hh][nt][r];
                    }
                } else {
                    float* out = xm.tap + (tk * H + h0 + hh) * (int64_t)P * N + (int64_t)(16 * w + l16) * N + 4 * g4;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(out + 16 * nt) = st[hh][nt];
                }
            }
        }
        __syncthreads();  // the previous sub-chunk's readers are done with the LDS tiles
        chunk_store<N, HPW, true, FWD, RAW>(sm.xs, sm.bs, sm.cs, sm.lw, sm.dtw, sm.ww, sm.ec, sm.alpha, rg, ad,
                                            cs_prev, tot, tid, &ds.fe, h0 + (tid >> 6), ah);
        if (REV && rsrc && tid < 64 * HPW) sm.rs[tid] = rg.rs;
        __syncthreads();
        if (sc + 1 < nsub) {
            const int64_t t1 = tbase + QS;
            chunk_load<N, HPW, true, REV, RAW>(
                rg, ad, tile_base<true, REV, RAW>(x, B, C, ds, dt0, b, L, xm.hx, G, N, xh0, g, t1, sc + 1, xm.rows), xm.hx,
                G, tid);
            load_rs(t1);
        }

        // ---- phase 1: C.B^T tiles, decayed per head -> LDS in fragment order ----------------
        for (int tt = w; tt < 10; tt += 4) {
            // tile tt = it (it + 1) / 2 + jt of the lower triangle, from arithmetic (no table lookup)
            const int it = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
            const int jt = tt - it * (it + 1) / 2;
            f32x4 gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
                Frag<bf16> a, bo;
                frag_load8<bf16>(a, &sm.bs[(16 * jt + l16) * BS + 32 * ks + 8 * g4]);
                frag_load8<bf16>(bo, &sm.cs[(16 * it + l16) * CS + 32 * ks + 8 * g4]);
                mma(gacc, a, bo);
            }
            const int i = 16 * it + l16, j0 = 16 * jt + 4 * g4;
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                f32x4 m;
                if (jt == it) {
                    // diagonal tile: every operand is read and every product formed, then the upper
                    // triangle is selected to zero (the exponent is capped at 0 so no lane forms an
                    // infinity); D_h joins the diagonal, so X^T M also yields the skip term D x
                    const float li = sm.lw[hh * QS + i];
                    const f32x4 lj = *reinterpret_cast<const f32x4*>(&sm.lw[hh * QS + j0]);
                    const f32x4 dj = *reinterpret_cast<const f32x4*>(&sm.dtw[hh * QS + j0]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = gacc[r] * fast_exp2(fminf(li - lj[r], 0.0f)) * dj[r];
                        m[r] = (j0 + r <= i ? v : 0.0f) + (!REV && j0 + r == i ? Dh[hh] : 0.0f);
                    }
                } else {  // below the diagonal: the separable factors of chunk_store
                    const float er = sm.ec[(hh * 4) * QS + i];
                    const f32x4 ej = *reinterpret_cast<const f32x4*>(&sm.ec[(hh * 4 + it) * QS + j0]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[r] = gacc[r] * er * ej[r];
                }
                *reinterpret_cast<bf16x4*>(&sm.mb[((hh * 16 + jt * 4 + it) * 64 + lane) * 4]) = cvt4(m);
            }
        }
        __syncthreads();

        // ---- phase 2: Y^T[p-tile w] = 2^l_i (S C^T) + X^T M  (M carries D on its diagonal) -------
        bf16x8 sa[HPW][NK];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) sa[hh][ks] = pack8(cvt4(st[hh][2 * ks]), cvt4(st[hh][2 * ks + 1]));
        }
        // X^T fragments of this wavefront's p-tile over token slots 32ks + 4g4 + r and
        // 32ks + 16 + 4g4 + r: read once, used by the in-chunk product here and, scaled, by the
        // state update of phase 3
        Frag<bf16> xf[2][HPW];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const bf16* xt = &sm.xs[hh * QS * XS];
                xf[ks][hh].v = pack8(tr_read(xt, 32 * ks + 4 * g4, 16 * w, XS, l16),
                                     tr_read(xt, 32 * ks + 16 + 4 * g4, 16 * w, XS, l16));
            }
        }
        const bool full = tbase + QS <= L;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = 16 * it + l16;
            f32x4 acc[HPW];
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) acc[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16* crow = &sm.cs[i * CS];
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
                Frag<bf16> bo;
                bo.v = pack8(*reinterpret_cast<const bf16x4*>(crow + 32 * ks + 4 * g4),
                             *reinterpret_cast<const bf16x4*>(crow + 32 * ks + 16 + 4 * g4));
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    Frag<bf16> a;
                    a.v = sa[hh][ks];
                    mma(acc[hh], a, bo);
                }
            }
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const float sc_i = fast_exp2(sm.lw[hh * QS + i]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[hh][r] *= sc_i;
            }
#pragma unroll
            for (int js = 0; js <= it / 2; ++js) {
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    Frag<bf16> bo;
                    const bf16* mt = &sm.mb[hh * 16 * 256];
                    bo.v = pack8(*reinterpret_cast<const bf16x4*>(&mt[(((2 * js) * 4 + it) * 64 + lane) * 4]),
                                 *reinterpret_cast<const bf16x4*>(&mt[(((2 * js + 1) * 4 + it) * 64 + lane) * 4]));
                    mma(acc[hh], xf[js][hh], bo);
                }
            }
            if (REV) {  // forward rows: y = s (C.S + in-chunk term) + D x, nothing for the padding tokens
                const int64_t f = L - 1 - (tbase + i);
                if (f < xm.rows) {
#pragma unroll
                    for (int hh = 0; hh < HPW; ++hh) {
                        const float s = rsrc ? sm.rs[hh * QS + i] : 1.0f;
                        const bf16x4 xv = *reinterpret_cast<const bf16x4*>(&sm.xs[(hh * QS + i) * XS + 16 * w + 4 * g4]);
                        bf16x4 o;
#pragma unroll
                        for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(fmaf(s, acc[hh][r], Dh[hh] * static_cast<float>(xv[r])));
                        *reinterpret_cast<bf16x4*>(y + ((b * xm.rows + f) * H + h0 + hh) * (int64_t)P + 16 * w + 4 * g4) = o;
                    }
                }
            } else if (full || tbase + i < L) {
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[hh][r]);
                    // a 32-bit byte offset from a scalar base at dstate 128 (measured 1.2-1.5% faster there and
                    // 2-3% slower at dstate 64 than the element offset)
                    if (N >= 128)
                        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(y + ((b * L + tbase) * H + h0) * (int64_t)P) +
                                                   (yo + (uint32_t)((16 * it * H + hh) * P)) * 2u) = o;
                    else
                        *reinterpret_cast<bf16x4*>(y + ((b * L + tbase) * H + h0) * (int64_t)P +
                                                   (yo + (uint32_t)((16 * it * H + hh) * P))) = o;
                }
            }
        }

        // ---- phase 3: S <- 2^(l_63) S + B^T (w x) ---------------------------------------------
        // With taps the state's decay is applied inside the first K step (ahead of it, the reversed
        // dstate-128 scan spilled registers).
        auto decay_state = [&]() {
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const float alpha = sm.alpha[hh];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) st[hh][nt][r] *= alpha;
                }
            }
        };
        if constexpr (!TAP) {  // (the same loop as decay_state, written out: the call form compiles differently)
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const float alpha = sm.alpha[hh];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) st[hh][nt][r] *= alpha;
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // token slots of this K step: 32ks + 4g4 + r (slots 0..3) and 32ks + 16 + 4g4 + r (slots 4..7)
            if constexpr (TAP) {  // hi + lo scaled operand; the B^T fragments in two halves (fewer live registers)
                if (ks == 0) decay_state();
                Frag<bf16> xw[HPW], xl[HPW];
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    const float* wv = &sm.ww[hh * QS + 32 * ks + 4 * g4];
                    const f32x4 w0 = {wv[0], wv[1], wv[2], wv[3]}, w1 = {wv[16], wv[17], wv[18], wv[19]};
                    const bf16x4 x0 = {xf[ks][hh].v[0], xf[ks][hh].v[1], xf[ks][hh].v[2], xf[ks][hh].v[3]};
                    const bf16x4 x1 = {xf[ks][hh].v[4], xf[ks][hh].v[5], xf[ks][hh].v[6], xf[ks][hh].v[7]};
                    const f32x4 v0 = __builtin_convertvector(x0, f32x4) * w0;
                    const f32x4 v1 = __builtin_convertvector(x1, f32x4) * w1;
                    const bf16x4 h0 = __builtin_convertvector(v0, bf16x4), h1 = __builtin_convertvector(v1, bf16x4);
                    xw[hh].v = pack8(h0, h1);
                    xl[hh].v = pack8(__builtin_convertvector(v0 - bf16x4_to_f32(h0), bf16x4),
                                     __builtin_convertvector(v1 - bf16x4_to_f32(h1), bf16x4));
                }
#pragma unroll
                for (int nb = 0; nb < NT; nb += NT / 2) {
                    Frag<bf16> a[NT / 2];
#pragma unroll
                    for (int q = 0; q < NT / 2; ++q)
                        a[q].v = pack8(tr_read(sm.bs, 32 * ks + 4 * g4, 16 * (nb + q), BS, l16),
                                       tr_read(sm.bs, 32 * ks + 16 + 4 * g4, 16 * (nb + q), BS, l16));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int q = 0; q < NT / 2; ++q) {
#pragma unroll
                        for (int hh = 0; hh < HPW; ++hh) {
                            mma(st[hh][nb + q], a[q], xw[hh]);
                            mma(st[hh][nb + q], a[q], xl[hh]);
                        }
                    }
                }
            } else {
                Frag<bf16> xw[HPW];
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    const float* wv = &sm.ww[hh * QS + 32 * ks + 4 * g4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        xw[hh].v[r] = static_cast<bf16>(static_cast<float>(xf[ks][hh].v[r]) * wv[r]);
                        xw[hh].v[4 + r] = static_cast<bf16>(static_cast<float>(xf[ks][hh].v[4 + r]) * wv[16 + r]);
                    }
                }
                Frag<bf16> a[NT];  // every B^T fragment of this K step in flight before the products
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    a[nt].v = pack8(tr_read(sm.bs, 32 * ks + 4 * g4, 16 * nt, BS, l16),
                                    tr_read(sm.bs, 32 * ks + 16 + 4 * g4, 16 * nt, BS, l16));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                    for (int hh = 0; hh < HPW; ++hh) mma(st[hh][nt], a[nt], xw[hh]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// chunk-state kernel: the state each chunk produces from zero (hi/lo)
// ---------------------------------------------------------------------------
template <int N, int HPW>
struct AggLds {
    bf16 xs[HPW * QS * XS];
    bf16 bs[QS * Strides<N>::BS];
    float ww[HPW * QS];  // 2^(l_end - l_j) dt_j: token j's weight in the chunk's end state
};

// registers -> LDS for the chunk-state kernel, and each token's weight in the state at the chunk's
// end (one wavefront per head).  FWD: the decay arrays restart at every sub-chunk, the sub-chunks are
// walked from the last, `after` holds the log2 decay from this sub-chunk's end to the chunk's end and
// tot accumulates the chunk's total.  Otherwise cs is cumulative over the chunk and cs_end is its
// value at the chunk's last position (flat past the sequence end, where dt is zero).
// RAW (with FWD): the steps and the sub-chunk's cumulative decay from the raw dt, as in chunk_store.
template <int N, int HPW, bool FWD, bool RAW = false>
__device__ __forceinline__ void state_store(bf16* xs, bf16* bsm, float* ww, const ChunkRegs<N, HPW, false>& rg,
                                            const ChunkAddr<N, HPW>& a, float& after, float cs_end, float& tot,
                                            int tid, const DtFront* fe = nullptr, int h = 0, float ah = 0.0f) {
    constexpr int RPI = BRows<N>::RPI, BS = Strides<N>::BS;
#pragma unroll
    for (int k = 0; k < 2 * HPW; ++k)
        *reinterpret_cast<uint4*>(xs + a.xl + (k >> 1) * QS * XS + (k & 1) * 32 * XS) = rg.x[k];
#pragma unroll
    for (int k = 0; k < N / 32; ++k) *reinterpret_cast<uint4*>(bsm + a.bl + k * RPI * BS) = rg.b[k];
    if (tid < 64 * HPW) {
        float cs = rg.cs, d = rg.dt;
        if (RAW) {
            float dec = 0.0f, inp = 0.0f;  // zero past the sequence end
            if (rg.cs != 0.0f) dt_front(*fe, h, ah, rg.dt, dec, inp);
            d = inp;
            cs = wave_incl_scan(dec * ah) * kLog2e;
        }
        float e;  // log2 decay from this token to the chunk's end
        if (FWD) {
            const float last = lane_read(cs, 63);
            e = after + (last - cs);
            after += last;
            tot += last;
        } else {
            e = cs_end - cs;
        }
        ww[(tid >> 6) * QS + (tid & 63)] = fast_exp2(e) * d;
    }
}

// Every token's contribution reaches the chunk's end through one weight, 2^(l_end - l_j) dt_j, so
// the state is a plain sum over the chunk's tokens: S = sum_j B_j (outer) (w_j x_j), accumulated in
// the MFMA registers with no per-sub-chunk decay of the partial state.  The sub-chunks are walked from
// the last to the first, which makes each sub-chunk's distance to the chunk's end known when its
// weights are formed.
// FWD: the forward's variant -- reads sub-chunk-local decay arrays and also writes each chunk's total
// log2 decay to totals (b, H, nC).  REV: the inputs are walked backwards (XMap::rows).  RAW (with FWD,
// forwards): the decays come from the raw dt (DtSrc::raw), formed per sub-chunk in registers.
template <int N, int HPW, bool FWD, bool REV = false, bool RAW = false>
__global__ void __launch_bounds__(256, 2)
chunk_state_fast_kernel(const bf16* __restrict__ x, const bf16* __restrict__ B, DtSrc ds, float* __restrict__ states,
                        float* __restrict__ totals, int64_t L, int H, int G, int Q, int64_t nC, uint32_t nitems,
                        XMap xm) {
    constexpr int NT = N / 16;
    constexpr int BS = Strides<N>::BS;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    AggLds<N, HPW>& sm = *reinterpret_cast<AggLds<N, HPW>*>(smem_raw);

    const int HP = H / HPW;
    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int hp = (int)(item % (uint32_t)HP);
    const int64_t c = (item / (uint32_t)HP) % (uint32_t)nC;
    const int64_t b = item / ((uint32_t)HP * (uint32_t)nC);
    const int h0 = hp * HPW;
    const int g = h0 / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index, in a scalar register
    const int64_t t0 = c * Q;
    const int64_t t_end = t0 + Q < L ? t0 + Q : L;
    const int nsub = (int)((t_end - t0 + QS - 1) / QS);

    f32x4 st[HPW][NT];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st[hh][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t nsubT = (L + QS - 1) / QS;
    static_assert(!RAW || (FWD && !REV), "raw decays: the forward's chunk state only");
    // dt/cs distance between heads (RAW: the raw dt's row length) and this chunk's first element
    const int64_t dt_head = RAW ? (int64_t)ds.H : FWD ? nsubT * QS : nC * Q;
    const int64_t dt0 = RAW   ? b * L * ds.H + h0
                        : FWD ? ((b * H + h0) * nsubT + c * (Q / QS)) * QS
                              : ((b * H + h0) * nC + c) * Q;
    const float ah = RAW && tid < 64 * HPW ? ds.A[h0 + (tid >> 6)] : 0.0f;  // A of this thread's head
    float after = 0.0f, tot = 0.0f, cs_end = 0.0f;
    if (!FWD && tid < 64 * HPW) cs_end = ds.cs[dt0 + (int64_t)(tid >> 6) * dt_head + (Q - 1)];
    const int xh0 = h0 / xm.div * xm.mul;  // the x heads of this head pair
    ChunkAddr<N, HPW> ad;
    chunk_addr<N, HPW, REV, RAW>(ad, xm.hx, G, dt_head, tid);
    ChunkRegs<N, HPW, false> rg;
    {
        const int64_t tl = t0 + (int64_t)(nsub - 1) * QS;
        chunk_load<N, HPW, false, REV, RAW>(
            rg, ad, tile_base<false, REV, RAW>(x, B, nullptr, ds, dt0, b, L, xm.hx, G, N, xh0, g, tl, nsub - 1, xm.rows),
            xm.hx, G, tid);
    }

    for (int sc = nsub - 1; sc >= 0; --sc) {
        __syncthreads();
        state_store<N, HPW, FWD, RAW>(sm.xs, sm.bs, sm.ww, rg, ad, after, cs_end, tot, tid, &ds.fe, h0 + (tid >> 6),
                                      ah);
        __syncthreads();
        if (sc > 0) {
            const int64_t t1 = t0 + (int64_t)(sc - 1) * QS;
            chunk_load<N, HPW, false, REV, RAW>(
                rg, ad, tile_base<false, REV, RAW>(x, B, nullptr, ds, dt0, b, L, xm.hx, G, N, xh0, g, t1, sc - 1, xm.rows),
                xm.hx, G, tid);
        }

#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            Frag<bf16> xh[HPW], xl[HPW];
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const bf16* xt = &sm.xs[hh * QS * XS];
                const bf16x4 lo4 = tr_read(xt, 32 * ks + 4 * g4, 16 * w, XS, l16);
                const bf16x4 hi4 = tr_read(xt, 32 * ks + 16 + 4 * g4, 16 * w, XS, l16);
                const float* wv = &sm.ww[hh * QS + 32 * ks + 4 * g4];
                const f32x4 w0 = {wv[0], wv[1], wv[2], wv[3]}, w1 = {wv[16], wv[17], wv[18], wv[19]};
                const f32x4 v0 = __builtin_convertvector(lo4, f32x4) * w0;
                const f32x4 v1 = __builtin_convertvector(hi4, f32x4) * w1;
                const bf16x4 h0 = __builtin_convertvector(v0, bf16x4), h1 = __builtin_convertvector(v1, bf16x4);
                xh[hh].v = pack8(h0, h1);
                xl[hh].v = pack8(__builtin_convertvector(v0 - bf16x4_to_f32(h0), bf16x4),
                                 __builtin_convertvector(v1 - bf16x4_to_f32(h1), bf16x4));
            }
            Frag<bf16> a[NT];  // every B^T fragment of this K step in flight before the products
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                a[nt].v = pack8(tr_read(sm.bs, 32 * ks + 4 * g4, 16 * nt, BS, l16),
                                tr_read(sm.bs, 32 * ks + 16 + 4 * g4, 16 * nt, BS, l16));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                for (int hh = 0; hh < HPW; ++hh) {
                    mma(st[hh][nt], a[nt], xh[hh]);
                    mma(st[hh][nt], a[nt], xl[hh]);
                }
            }
        }
    }
    // a ragged last chunk ends at position Q-1 all the same: its padded tokens have dt = 0 and decay 1
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        float* out = states + ((b * nC + c) * H + h0 + hh) * (int64_t)P * N + (int64_t)(16 * w + l16) * N + 4 * g4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(out + 16 * nt) = st[hh][nt];
    }
    if (FWD && tid < 64 * HPW && lane == 0) totals[(b * H + h0 + w) * nC + c] = tot;
}

// ---------------------------------------------------------------------------
// the forward's decay arrays: for every 64-token sub-chunk and head,
//   dtl[b,h,s,i] = dt[b, 64s+i, h],   lw[b,h,s,i] = log2(e) sum_{k<=i} dt[b,64s+k,h] A[h]
// (dt after the front-end: the input step in dtl, the decay step in lw)
// (the in-chunk cumulative sum with the chunk length set to 64).  One workgroup
// per (b, s): the (64 x H) block of dt is contiguous, read coalesced through LDS
// in blocks of 64 heads; each wavefront then scans one head at a time.
// ---------------------------------------------------------------------------
constexpr int kDecayHB = 64;  // heads per LDS block

// Steps of the backward's scans (BWD): kernel head h reads dt head h / hdiv of a (b, Ls, H / hdiv) array
// (the half-heads of a transposed scan share their head's steps and A); with rev the kernel's token t
// (of L) takes the decay step of dt row L - t -- the reversed adjoint recurrence applies the decay of the
// token after t, so the first real token (t = L - Ls) and the padding before it take none -- and with
// unit the input step is 1.  Without BWD: the forward's arrays (Ls = L, hdiv = 1, no rev, no unit).
struct DecaySrc {
    int64_t Ls;
    int hdiv, rev, unit;
};

template <bool BWD>
__device__ __forceinline__ void subchunk_decay_body(const DtFront& fe, const bf16* __restrict__ dt,
                                                    const float* __restrict__ A, float* __restrict__ dtl,
                                                    float* __restrict__ lw, int64_t L, int H, uint32_t nitems,
                                                    const DecaySrc& src, uint32_t block) {
    __shared__ float blk[QS][kDecayHB + 1];
    __shared__ bool vok[QS][kDecayHB + 1];  // position inside the sequence
    const int64_t nsubT = (L + QS - 1) / QS;
    const uint32_t item = xcd_remap(block, nitems);
    const int64_t sub = item % (uint64_t)nsubT;
    const int64_t b = item / (uint64_t)nsubT;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int64_t t0 = sub * QS;
    const int Hs = BWD ? H / src.hdiv : H;
    for (int hb = 0; hb < H; hb += kDecayHB) {
        const int nh = H - hb < kDecayHB ? H - hb : kDecayHB;
        __syncthreads();
        constexpr int KL = QS * kDecayHB / 256;
        bf16 v[KL];  // all loads in flight before the first use
#pragma unroll
        for (int k = 0; k < KL; ++k) {
            const int e = tid + 256 * k, t = e / kDecayHB, hh = e % kDecayHB;
            bool ok = hh < nh && t0 + t < L;  // load a valid element regardless, then select
            int64_t row = t0 + t;
            int hs = hb + hh;
            if (BWD) {
                row = src.rev ? L - (t0 + t) : t0 + t;
                ok = ok && row < src.Ls;
                hs = (hb + hh) / src.hdiv;
            }
            v[k] = dt[ok ? (b * (BWD ? src.Ls : L) + row) * Hs + hs : 0];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < KL; ++k) {
            const int e = tid + 256 * k, t = e / kDecayHB, hh = e % kDecayHB;
            bool ok = hh < nh && t0 + t < L;
            if (BWD) ok = ok && (src.rev ? L - (t0 + t) : t0 + t) < src.Ls;
            blk[t][hh] = ok ? to_f32(v[k]) : 0.0f;
            vok[t][hh] = ok;
        }
        __syncthreads();
        for (int hh = w; hh < nh; hh += 4) {
            const int h = hb + hh;
            const float ah = A[BWD ? h / src.hdiv : h];
            float dec = 0.0f, d = 0.0f;  // decay and input steps; zero past L
            if (vok[lane][hh]) dt_front(fe, h, ah, blk[lane][hh], dec, d);
            if (BWD && src.unit) d = t0 + lane < L ? 1.0f : 0.0f;
            const float incl = wave_incl_scan(dec * ah);  // DPP steps, no LDS permutes
            const int64_t o = ((b * H + h) * nsubT + sub) * QS + lane;
            dtl[o] = d;
            lw[o] = incl * kLog2e;
        }
    }
}

template <bool BWD>
__global__ void __launch_bounds__(256) subchunk_decay_kernel(DtFront fe, const bf16* __restrict__ dt,
                                                             const float* __restrict__ A, float* __restrict__ dtl,
                                                             float* __restrict__ lw, int64_t L, int H,
                                                             uint32_t nitems, DecaySrc src) {
    subchunk_decay_body<BWD>(fe, dt, A, dtl, lw, L, H, nitems, src, blockIdx.x);
}

// several sets of the backward's decay arrays in one launch: set blockIdx.y, workgroups past its count idle
struct DecayJob {
    float *dtl, *lw;
    int64_t L;
    int H;
    uint32_t nitems;
    DecaySrc src;
};
struct DecayJobs {
    DecayJob j[3];
};

__global__ void __launch_bounds__(256) subchunk_decay_jobs_kernel(const bf16* __restrict__ dt, const float* __restrict__ A,
                                                                  DecayJobs jobs) {
    const DecayJob& jb = jobs.j[blockIdx.y];
    if (blockIdx.x >= jb.nitems) return;
    const DtFront none{nullptr, 0, 0, 0, 0.0f, 0.0f};
    subchunk_decay_body<true>(none, dt, A, jb.dtl, jb.lw, jb.L, jb.H, jb.nitems, jb.src, blockIdx.x);
}

// Reading the inputs backwards (XMap::rows > 0) is a variant of the kernels with sub-chunk-local decay
// arrays (FWD); it needs whole 64-token tiles (L a multiple of 64) so that every tile's first input row
// lies inside the batch row.  Taps need a spacing that is a multiple of the sub-chunk (every tap position
// starts a sub-chunk).
inline bool rev_ok(const Shape& s, const XMap& xm) { return xm.rows >= 0 && xm.rows <= s.L && s.L % QS == 0; }
inline bool tap_ok(const Shape& s, const XMap& xm) { return xm.tapq > 0 && xm.tapq % QS == 0 && s.Q % QS == 0; }

template <int N, int HPW, bool FWD>
hipError_t launch_state_fast(const Shape& s, const bf16* x, const bf16* B, const DtSrc& ds, float* states,
                             float* totals, const XMap& xm, hipStream_t st) {
    const uint32_t nitems = (uint32_t)(s.b * s.nC * (s.H / HPW));
    if (nitems == 0) return hipSuccess;
    const size_t lds = sizeof(AggLds<N, HPW>);
    const bool rev = xm.rows > 0, raw = ds.raw != nullptr;
    if (rev && (!FWD || !rev_ok(s, xm))) return hipErrorInvalidValue;
    if (raw && (!FWD || rev)) return hipErrorInvalidValue;
    const void* fn = rev   ? (const void*)chunk_state_fast_kernel<N, HPW, true, true>
                     : raw ? (const void*)chunk_state_fast_kernel<N, HPW, true, false, true>
                           : (const void*)chunk_state_fast_kernel<N, HPW, FWD>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (rev)
        hipLaunchKernelGGL((chunk_state_fast_kernel<N, HPW, true, true>), dim3(nitems), dim3(256), lds, st, x, B, ds,
                           states, totals, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    else if (raw)
        hipLaunchKernelGGL((chunk_state_fast_kernel<N, HPW, true, false, true>), dim3(nitems), dim3(256), lds, st, x,
                           B, ds, states, totals, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    else
        hipLaunchKernelGGL((chunk_state_fast_kernel<N, HPW, FWD>), dim3(nitems), dim3(256), lds, st, x, B, ds, states,
                           totals, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    return hipGetLastError();
}

template <int N, int HPW, bool FWD>
hipError_t launch_scan_fast(const Shape& s, const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                            const float* start, const float* D, bf16* y, const XMap& xm, hipStream_t st) {
    const uint32_t nitems = (uint32_t)(s.b * s.nC * (s.H / HPW));
    if (nitems == 0) return hipSuccess;
    const size_t lds = sizeof(ScanLds<N, HPW>);
    const bool rev = xm.rows > 0, tap = xm.tap != nullptr, raw = ds.raw != nullptr;
    if (rev && (!FWD || !rev_ok(s, xm))) return hipErrorInvalidValue;
    if (raw && (!FWD || rev || tap || xm.start_tr)) return hipErrorInvalidValue;
    if (tap && (!FWD || !tap_ok(s, xm))) return hipErrorInvalidValue;
    if (tap && (xm.tap_tr != 0) == rev) return hipErrorInvalidValue;  // taps: reversed, or transposed forwards
    if (xm.tap_tr && (!tap || xm.tap_tr > 2 || s.H % xm.tap_tr != 0)) return hipErrorInvalidValue;
    if (xm.start_tr && !rev) return hipErrorInvalidValue;
    const void* fn = tap   ? (rev ? (const void*)chunk_scan_fast_kernel<N, HPW, true, true, true>
                                  : (const void*)chunk_scan_fast_kernel<N, HPW, true, false, true, true>)
                     : rev ? (const void*)chunk_scan_fast_kernel<N, HPW, true, true, false>
                     : raw ? (const void*)chunk_scan_fast_kernel<N, HPW, true, false, false, false, true>
                           : (const void*)chunk_scan_fast_kernel<N, HPW, FWD>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (tap && rev)
        hipLaunchKernelGGL((chunk_scan_fast_kernel<N, HPW, true, true, true>), dim3(nitems), dim3(256), lds, st, x, B,
                           C, ds, start, D, y, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    else if (tap)
        hipLaunchKernelGGL((chunk_scan_fast_kernel<N, HPW, true, false, true, true>), dim3(nitems), dim3(256), lds, st,
                           x, B, C, ds, start, D, y, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    else if (rev)
        hipLaunchKernelGGL((chunk_scan_fast_kernel<N, HPW, true, true, false>), dim3(nitems), dim3(256), lds, st, x, B,
                           C, ds, start, D, y, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    else if (raw)
        hipLaunchKernelGGL((chunk_scan_fast_kernel<N, HPW, true, false, false, false, true>), dim3(nitems), dim3(256),
                           lds, st, x, B, C, ds, start, D, y, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    else
        hipLaunchKernelGGL((chunk_scan_fast_kernel<N, HPW, FWD>), dim3(nitems), dim3(256), lds, st, x, B, C, ds, start,
                           D, y, s.L, (int)s.H, (int)s.G, (int)s.Q, s.nC, nitems, xm);
    return hipGetLastError();
}

// wide-state kernels (dstate 256 and 512, one head per workgroup), wide.hip
template <bool FWD>
hipError_t state_wide(const Shape& s, const bf16* x, const bf16* B, const DtSrc& ds, float* states, float* totals,
                      hipStream_t st);
template <bool FWD>
hipError_t scan_wide(const Shape& s, const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                     const float* start, const float* D, bf16* y, hipStream_t st);

// dispatch over (N, heads per workgroup)
template <bool FWD>
hipError_t state_dispatch(const Shape& s, const bf16* x, const bf16* B, const DtSrc& ds, float* states,
                          float* totals, hipStream_t st, const XMap* xm = nullptr);
template <bool FWD>
hipError_t scan_dispatch(const Shape& s, const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                         const float* start, const float* D, bf16* y, hipStream_t st, const XMap* xm = nullptr);

}  // namespace fz

bool fast_chunk_supported(const Shape& s) {
    return s.io == 1 && s.P == 64 && (s.N == 64 || s.N == 128 || s.N == 256 || s.N == 512) && s.Q % 64 == 0;
}

// heads per workgroup: two when both heads of every pair read the same group (dstate <= 128;
// the wide-state kernels in wide.hip take one head per workgroup)
static int fast_hpw(const Shape& s) { return s.N <= 128 && (s.H / s.G) % 2 == 0 ? 2 : 1; }

int fast_heads_per_wg(const Shape& s) { return fast_hpw(s); }

int fast_forward_chunk(const Shape& s) {
    // the largest power of two (<= 4096 tokens) that still gives enough (b, chunk, head-pair) work items
    const int64_t items_per_token = s.b * s.H / fast_hpw(s);
    int64_t q0 = 4096;
    while (q0 > 256 && items_per_token * s.L / q0 < 1024) q0 /= 2;
    // dstate <= 128: refine over the multiples of 64 in [q0/2, 2 q0] by
    // the workgroup rounds of the two chunk kernels (two resident per CU on the 256 CUs of gfx950).
    // A round costs one chunk length of sub-chunk steps; a last round with at most one workgroup per
    // CU runs about 1.6x faster per workgroup (measured); each chunk adds a state round trip through
    // HBM, worth about 8 tokens.  At 2.7B/64K this picks 2624 (1000 workgroups, two full rounds)
    // over 2048 (1280, two and a half rounds): 0.794 against 0.811 ms.
    // Below one round of workgroups only smaller chunks are tried (more workgroups in flight): at
    // 2.7B/1K this picks 192 over 256 (0.050 against 0.054 ms); below a quarter round the anchor stays.
    constexpr int64_t kSlots = 2 * 256;
    constexpr double kLoneSpeed = 1.0 / 1.6, kChunkCost = 8.0;
    const int64_t items0 = items_per_token * ((s.L + q0 - 1) / q0);
    if (s.N > 128 || items0 < kSlots / 4) return (int)q0;
    const int64_t qmax = items0 >= kSlots ? 2 * q0 : q0;
    int64_t best = q0;
    double best_cost = 0.0;
    for (int64_t q = (q0 / 2 + 63) / 64 * 64; q <= qmax && q <= 4096; q += 64) {
        if (q < 128) continue;
        const int64_t nC = (s.L + q - 1) / q, items = items_per_token * nC;
        const int64_t full = items / kSlots, rest = items % kSlots;
        const double rounds = (double)full + (rest == 0 ? 0.0 : (rest <= kSlots / 2 ? kLoneSpeed : 1.0));
        const double cost = rounds * (double)(q < s.L ? q : s.L) + kChunkCost * (double)nC;
        if (best_cost == 0.0 || cost < best_cost) best_cost = cost, best = q;
    }
    return (int)best;
}

namespace fz {

template <bool FWD>
hipError_t state_dispatch(const Shape& s, const bf16* x, const bf16* B, const DtSrc& ds, float* states,
                          float* totals, hipStream_t st, const XMap* xm) {
    if (s.N >= 256) {
        if (xm) return hipErrorInvalidValue;  // the wide kernels read x in place, forwards
        return state_wide<FWD>(s, x, B, ds, states, totals, st);
    }
    const XMap id{(int)s.H, 1, 1, 0};
    const XMap& m = xm ? *xm : id;
    const bool pair = fast_hpw(s) == 2;
    if (s.N == 128)
        return pair ? launch_state_fast<128, 2, FWD>(s, x, B, ds, states, totals, m, st)
                    : launch_state_fast<128, 1, FWD>(s, x, B, ds, states, totals, m, st);
    return pair ? launch_state_fast<64, 2, FWD>(s, x, B, ds, states, totals, m, st)
                : launch_state_fast<64, 1, FWD>(s, x, B, ds, states, totals, m, st);
}

template <bool FWD>
hipError_t scan_dispatch(const Shape& s, const bf16* x, const bf16* B, const bf16* C, const DtSrc& ds,
                         const float* start, const float* D, bf16* y, hipStream_t st, const XMap* xm) {
    if (s.N >= 256) {
        if (xm) return hipErrorInvalidValue;  // the wide kernels read x in place, forwards
        return scan_wide<FWD>(s, x, B, C, ds, start, D, y, st);
    }
    const XMap id{(int)s.H, 1, 1, 0};
    const XMap& m = xm ? *xm : id;
    const bool pair = fast_hpw(s) == 2;
    if (s.N == 128)
        return pair ? launch_scan_fast<128, 2, FWD>(s, x, B, C, ds, start, D, y, m, st)
                    : launch_scan_fast<128, 1, FWD>(s, x, B, C, ds, start, D, y, m, st);
    return pair ? launch_scan_fast<64, 2, FWD>(s, x, B, C, ds, start, D, y, m, st)
                : launch_scan_fast<64, 1, FWD>(s, x, B, C, ds, start, D, y, m, st);
}

}  // namespace fz

hipError_t launch_chunk_state_fast(const Shape& s, const void* x, const void* B, const float* dt_t, const float* cs,
                                   float* states, hipStream_t st, const XMap* xm) {
    const fz::DtSrc ds{dt_t, cs};
    return fz::state_dispatch<false>(s, (const bf16*)x, (const bf16*)B, ds, states, nullptr, st, xm);
}

hipError_t launch_chunk_scan_fast(const Shape& s, const void* x, const void* B, const void* C, const float* dt_t,
                                  const float* cs, const float* start, const float* D, void* y, hipStream_t st,
                                  const XMap* xm) {
    const fz::DtSrc ds{dt_t, cs};
    return fz::scan_dispatch<false>(s, (const bf16*)x, (const bf16*)B, (const bf16*)C, ds, start, D, (bf16*)y, st,
                                    xm);
}

hipError_t launch_chunk_state_sub(const Shape& s, const void* x, const void* B, const float* dtl, const float* lw,
                                  float* states, float* totals, hipStream_t st, const XMap* xm) {
    if (s.N >= 256) return hipErrorInvalidValue;
    const fz::DtSrc ds{dtl, lw};
    return fz::state_dispatch<true>(s, (const bf16*)x, (const bf16*)B, ds, states, totals, st, xm);
}

hipError_t launch_chunk_scan_sub(const Shape& s, const void* x, const void* B, const void* C, const float* dtl,
                                 const float* lw, const float* start, const float* D, void* y, hipStream_t st,
                                 const XMap* xm) {
    if (s.N >= 256) return hipErrorInvalidValue;
    const fz::DtSrc ds{dtl, lw};
    return fz::scan_dispatch<true>(s, (const bf16*)x, (const bf16*)B, (const bf16*)C, ds, start, D, (bf16*)y, st, xm);
}

hipError_t launch_subchunk_decay_bwd_sets(const DecaySet* sets, int nsets, const void* dt, const float* A,
                                          hipStream_t st) {
    if (nsets < 1 || nsets > 3) return hipErrorInvalidValue;
    fz::DecayJobs jobs{};
    uint32_t gx = 0;
    for (int k = 0; k < nsets; ++k) {
        const DecaySet& d = sets[k];
        if (d.hdiv < 1 || d.H % d.hdiv) return hipErrorInvalidValue;
        const uint32_t n = (uint32_t)(d.b * ((d.L + fz::QS - 1) / fz::QS));
        jobs.j[k] = fz::DecayJob{d.dtl, d.lw, d.L, d.H, n, fz::DecaySrc{d.Ls, d.hdiv, d.rev ? 1 : 0, d.unit ? 1 : 0}};
        gx = n > gx ? n : gx;
    }
    if (gx == 0) return hipSuccess;
    hipLaunchKernelGGL(fz::subchunk_decay_jobs_kernel, dim3(gx, (unsigned)nsets), dim3(256), 0, st, (const bf16*)dt, A,
                       jobs);
    return hipGetLastError();
}

// The chunk kernels form the decays from the raw dt themselves at dstate <= 128 when the forward is short
// (at most 2^20 token-heads): that saves the decay pass's launch, which dominates there (2.7B heads at
// 1K and 4K tokens: 40.6 and 73.4 against 48.5 and 81.5 us; the 130M shape: 56.9 against 59.9 us), while
// on long inputs the pass is cheaper than the in-kernel work (2.7B heads at 64K tokens: 0.763 against
// 0.753 ms).
static bool forward_raw_decay(const Shape& s) { return s.N <= 128 && s.b * s.L * s.H <= ((int64_t)1 << 20); }

FastFwdLayout fast_forward_layout(const Shape& s) {
    auto a256 = [](size_t v) { return (v + 255) / 256 * 256; };
    FastFwdLayout f;
    // the decay pass's arrays unless the chunk kernels form the decays themselves
    const size_t pos = forward_raw_decay(s) ? 0 : (size_t)(s.b * s.H * ((s.L + fz::QS - 1) / fz::QS) * fz::QS) * 4;
    f.dtl = 0;
    f.lw = a256(pos);
    f.states = f.lw + a256(pos);
    f.totals = f.states + a256((size_t)(s.b * s.nC * s.H * s.P * s.N) * 4);
    f.total = f.totals + a256((size_t)(s.b * s.H * s.nC) * 4);
    return f;
}

hipError_t launch_forward_fast(const Shape& s, const DtFront& fe, const void* x, const void* dt, const float* A,
                               const void* B,
                               const void* C, const float* D, const float* h0, void* y, float* final_state,
                               void* workspace, hipStream_t st) {
    const FastFwdLayout f = fast_forward_layout(s);
    char* ws = static_cast<char*>(workspace);
    float* dtl = reinterpret_cast<float*>(ws + f.dtl);
    float* lw = reinterpret_cast<float*>(ws + f.lw);
    float* states = reinterpret_cast<float*>(ws + f.states);
    float* totals = reinterpret_cast<float*>(ws + f.totals);
    const bf16 *xb = (const bf16*)x, *bb = (const bf16*)B, *cb = (const bf16*)C;
    fz::DtSrc ds{dtl, lw};
    hipError_t e;
    if (forward_raw_decay(s)) {
        ds = fz::DtSrc{nullptr, nullptr, (const bf16*)dt, A, fe, (int)s.H};
    } else {
        const uint32_t ndec = (uint32_t)(s.b * ((s.L + fz::QS - 1) / fz::QS));
        hipLaunchKernelGGL(fz::subchunk_decay_kernel<false>, dim3(ndec), dim3(256), 0, st, fe, (const bf16*)dt, A,
                           dtl, lw, s.L, (int)s.H, ndec, fz::DecaySrc{s.L, 1, 0, 0});
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = fz::state_dispatch<true>(s, xb, bb, ds, states, totals, st);
    if (e != hipSuccess) return e;
    // the pass reads one total per chunk: a chunk of "length 1" in its indexing
    Shape s1 = s;
    s1.Q = 1;
    e = launch_state_passing(s1, states, totals, h0, final_state, st);
    if (e != hipSuccess) return e;
    return fz::scan_dispatch<true>(s, xb, bb, cb, ds, states, D, (bf16*)y, st);
}

}  // namespace ssd
