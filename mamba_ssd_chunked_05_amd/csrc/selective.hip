// selective.hip -- Mamba-1 selective scan: per-channel diagonal state with a
// per-entry decay rate A[d, n], discretised in-kernel ("3.3 Hardware-Aware
// algorithms and GPU memory hierarchy optimisation", section 2.1: abar =
// exp(delta A); zero-order hold bbar = (delta A)^-1 (exp(delta A) - 1) delta B,
// or delta B), scanned and read out through C in one fused pass (section 3:
// load, discretise, scan, output projection, with only y written back).
//
// Work mapping: a workgroup owns 16 channels of one batch row and one
// sequence segment; lane (c, l) of the 256 threads holds the state entries
// n = l, l + 16, .. (N / 16 of them) of channel c in registers and walks the
// segment token by token.  Each 64-token tile of x, delta, B and C is staged
// once in LDS as fp32, transposed so that a lane reads four consecutive
// tokens with one 16-byte load; the delta front-end (bias, softplus, clamp)
// runs once per (token, channel) while staging.  The output sum over n is a
// butterfly over the 16 lanes of a channel that leaves token i of each
// 16-token group in lane i, so no lane reduces more than it keeps.
//
// Sequence segments (associativity of the first-order recurrence, section
// 4.1; the per-tile carried initial state of section 5.1): with fewer
// channels than the chip has SIMDs, the sequence is cut into segments.  A
// first pass computes each segment's end state from zero and the sum of its
// steps, a carry pass chains them in segment order
//   start[s + 1] = exp(A sum_{t in s} delta_t) start[s] + local[s],
// and the output pass rescans every segment from its start state.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace sel {

constexpr int TT = 64;      // tokens per LDS tile
constexpr int TS = TT + 4;  // LDS row stride in floats (rows of different lanes fall in different banks)
constexpr int CB = 16;      // channels per workgroup
constexpr int YS = CB + 1;  // output tile row stride

struct Args {
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;
    float* seg_states;  // (b, nseg - 1, Dc, N): local end states, then the carried start states
    float* seg_sums;    // (b, nseg - 1, Dc): sum of the steps over each segment
    void* y;
    float* final_state;
    DtFront fe;
    int64_t L, Lseg;
    int Dc, G, nseg;
};

template <int N>
struct Lds {
    float xs[CB * TS];
    float ds[CB * TS];
    float bs[N * TS];
    float cs[N * TS];
    float ys[TT * YS];
};

template <class T>
struct Io;
template <>
struct Io<float> {
    static constexpr int per16 = 4;  // elements per 16-byte piece
    __device__ static void unpack(const uint4& v, float* o) {
        o[0] = __uint_as_float(v.x), o[1] = __uint_as_float(v.y), o[2] = __uint_as_float(v.z),
        o[3] = __uint_as_float(v.w);
    }
};
template <>
struct Io<bf16> {
    static constexpr int per16 = 8;
    __device__ static void unpack(const uint4& v, float* o) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

// 16-byte pieces of one tile: x and delta rows (CB channels), then B and C rows (N entries)
template <class T, int N>
struct Pieces {
    static constexpr int PX = CB / Io<T>::per16;  // pieces per x / delta row
    static constexpr int PB = N / Io<T>::per16;   // pieces per B / C row
    static constexpr int NXD = 2 * TT * PX;
    static constexpr int NBC = 2 * TT * PB;
    static constexpr int KXD = NXD / 256, KBC = NBC / 256;  // per thread
    static_assert(NXD % 256 == 0 && NBC % 256 == 0, "tile pieces must split evenly over 256 threads");
};

template <class T, int N>
struct Stage {
    uint4 xd[Pieces<T, N>::KXD];
    uint4 bc[Pieces<T, N>::KBC];
};

struct Tile {
    int64_t b, t0;  // batch row, first token of the tile
    int last;       // last valid row of the tile (tokens past the segment end are padding)
};

// global -> registers (rows past `last` read row `last` and are zeroed when stored)
template <class T, int N>
__device__ __forceinline__ void stage_load(Stage<T, N>& st, const Args& a, const Tile& tl, int c0, int g, int tid) {
    using PC = Pieces<T, N>;
    const T* xg = static_cast<const T*>(a.x);
    const T* dg = static_cast<const T*>(a.delta);
    const T* bg = static_cast<const T*>(a.B);
    const T* cg = static_cast<const T*>(a.C);
#pragma unroll
    for (int k = 0; k < PC::KXD; ++k) {
        const int i = tid + 256 * k;
        const bool isd = i >= TT * PC::PX;
        const int j = isd ? i - TT * PC::PX : i;
        const int r = j / PC::PX, col = (j % PC::PX) * Io<T>::per16;
        const int rr = r <= tl.last ? r : tl.last;
        const T* base = isd ? dg : xg;
        st.xd[k] = *reinterpret_cast<const uint4*>(base + (tl.b * a.L + tl.t0 + rr) * a.Dc + c0 + col);
    }
#pragma unroll
    for (int k = 0; k < PC::KBC; ++k) {
        const int i = tid + 256 * k;
        const bool isc = i >= TT * PC::PB;
        const int j = isc ? i - TT * PC::PB : i;
        const int r = j / PC::PB, col = (j % PC::PB) * Io<T>::per16;
        const int rr = r <= tl.last ? r : tl.last;
        const T* base = isc ? cg : bg;
        st.bc[k] = *reinterpret_cast<const uint4*>(base + ((tl.b * a.L + tl.t0 + rr) * a.G + g) * N + col);
    }
}

// registers -> LDS, transposed to [row][token]; the step goes through the front-end here
template <class T, int N>
__device__ __forceinline__ void stage_store(Lds<N>& sm, const Stage<T, N>& st, const Args& a, const Tile& tl,
                                            int c0, int tid) {
    using PC = Pieces<T, N>;
    constexpr int E = Io<T>::per16;
#pragma unroll
    for (int k = 0; k < PC::KXD; ++k) {
        const int i = tid + 256 * k;
        const bool isd = i >= TT * PC::PX;
        const int j = isd ? i - TT * PC::PX : i;
        const int r = j / PC::PX, col = (j % PC::PX) * E;
        const bool ok = r <= tl.last;
        float v[E];
        Io<T>::unpack(st.xd[k], v);
        if (isd) {  // wave-uniform: the x and delta ranges are whole wavefronts
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float dec, inp;
                dt_front(a.fe, c0 + col + e, 0.0f, v[e], dec, inp);
                sm.ds[(col + e) * TS + r] = ok ? dec : 0.0f;  // padding tokens: zero step, state unchanged
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) sm.xs[(col + e) * TS + r] = ok ? v[e] : 0.0f;
        }
    }
#pragma unroll
    for (int k = 0; k < PC::KBC; ++k) {
        const int i = tid + 256 * k;
        const bool isc = i >= TT * PC::PB;
        const int j = isc ? i - TT * PC::PB : i;
        const int r = j / PC::PB, col = (j % PC::PB) * E;
        const bool ok = r <= tl.last;
        float v[E];
        Io<T>::unpack(st.bc[k], v);
        float* dst = isc ? sm.cs : sm.bs;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[(col + e) * TS + r] = ok ? v[e] : 0.0f;
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// v[j] holds this lane's partial for token j of 16; returns the sum over the 16 lanes of the row
// for token (lane % 16): four exchange steps, each keeping half of the remaining tokens
__device__ __forceinline__ float row_transpose_sum(float (&v)[16], int l16) {
    // partner i ^ 15 (row mirror): keep the half of the tokens named by bit 3
    const bool b3 = l16 & 8, b2 = l16 & 4, b1 = l16 & 2, b0 = l16 & 1;
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float keep = b3 ? v[j + 8] : v[j], send = b3 ? v[j] : v[j + 8];
        w[j] = keep + dpp<0x140>(send);
    }
    // partner i ^ 7 (half-row mirror), bit 2
    float u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float keep = b2 ? w[j + 4] : w[j], send = b2 ? w[j] : w[j + 4];
        u[j] = keep + dpp<0x141>(send);
    }
    // partner i ^ 3 (quad mirror, quad_perm 3,2,1,0), bit 1
    float q[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float keep = b1 ? u[j + 2] : u[j], send = b1 ? u[j] : u[j + 2];
        q[j] = keep + dpp<0x1B>(send);
    }
    // partner i ^ 1 (quad_perm 1,0,3,2), bit 0
    const float keep = b0 ? q[1] : q[0], send = b0 ? q[0] : q[1];
    return keep + dpp<0xB1>(send);
}

template <class T, int N, bool ZOH, bool OUT>
__global__ void __launch_bounds__(256) selective_scan_kernel(Args a, uint32_t nitems) {
    constexpr int SPT = N / 16;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Lds<N>& sm = *reinterpret_cast<Lds<N>*>(smem_raw);

    const int nblk = a.Dc / CB;
    const int nsegk = OUT ? a.nseg : a.nseg - 1;  // the first pass skips the last segment
    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int cblk = (int)(item % (uint32_t)nblk);
    const int seg = (int)((item / (uint32_t)nblk) % (uint32_t)nsegk);
    const int64_t b = item / ((uint32_t)nblk * (uint32_t)nsegk);
    const int c0 = cblk * CB;
    const int g = c0 / (a.Dc / a.G);
    const int tid = threadIdx.x, cl = tid >> 4, l16 = tid & 15;
    const int c = c0 + cl;
    const int64_t s0 = (int64_t)seg * a.Lseg;
    const int64_t s1 = s0 + a.Lseg < a.L ? s0 + a.Lseg : a.L;

    // per-lane constants of the state entries n = l16 + 16 s
    float a2[SPT], ia[SPT], za[SPT], h[SPT];
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
        const float Av = a.A[(int64_t)c * N + l16 + 16 * s];
        a2[s] = Av * kLog2e;
        ia[s] = Av != 0.0f ? 1.0f / Av : 0.0f;  // zero-order hold factor (e - 1) / A, limit delta at A = 0
        za[s] = Av != 0.0f ? 0.0f : 1.0f;
    }
    const float Dd = (OUT && a.D) ? a.D[c] : 0.0f;
    const int64_t sidx = ((b * (a.nseg - 1) + seg) * a.Dc + c) * (int64_t)N;  // this segment's slot
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
        float v = 0.0f;
        if (OUT) {
            if (seg == 0)
                v = a.h0 ? a.h0[(b * a.Dc + c) * (int64_t)N + l16 + 16 * s] : 0.0f;
            else
                v = a.seg_states[sidx - (int64_t)a.Dc * N + l16 + 16 * s];  // carried start of this segment
        }
        h[s] = v;
    }
    float dsum = 0.0f;

    Stage<T, N> st;
    Tile tl{b, s0, (int)(s1 - s0 - 1 < TT - 1 ? s1 - s0 - 1 : TT - 1)};
    stage_load<T, N>(st, a, tl, c0, g, tid);
    for (int64_t t0 = s0; t0 < s1; t0 += TT) {
        tl.t0 = t0;
        tl.last = (int)(s1 - t0 - 1 < TT - 1 ? s1 - t0 - 1 : TT - 1);
        __syncthreads();  // the previous tile's readers are done
        stage_store<T, N>(sm, st, a, tl, c0, tid);
        __syncthreads();
        if (t0 + TT < s1) {
            Tile nt{b, t0 + TT, (int)(s1 - t0 - TT - 1 < TT - 1 ? s1 - t0 - TT - 1 : TT - 1)};
            stage_load<T, N>(st, a, nt, c0, g, tid);
        }
        const float* drow = &sm.ds[cl * TS];
        const float* xrow = &sm.xs[cl * TS];
#pragma unroll 1
        for (int t16 = 0; t16 < TT; t16 += 16) {
            float p[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int tq = t16 + 4 * q4;
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(drow + tq);
                const f32x4 x4 = *reinterpret_cast<const f32x4*>(xrow + tq);
                f32x4 b4[SPT], c4[SPT];
#pragma unroll
                for (int s = 0; s < SPT; ++s) {
                    b4[s] = *reinterpret_cast<const f32x4*>(&sm.bs[(l16 + 16 * s) * TS + tq]);
                    if (OUT) c4[s] = *reinterpret_cast<const f32x4*>(&sm.cs[(l16 + 16 * s) * TS + tq]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dl = d4[r], xv = x4[r];
                    if (!OUT) dsum += dl;
                    const float dx = dl * xv;
                    float acc = 0.0f;
#pragma unroll
                    for (int s = 0; s < SPT; ++s) {
                        const float e = fast_exp2(dl * a2[s]);
                        float u;
                        if (ZOH) {
                            const float f = fmaf(dl, za[s], fmaf(e, ia[s], -ia[s]));  // (e - 1) / A
                            u = f * (b4[s][r] * xv);
                        } else {
                            u = dx * b4[s][r];
                        }
                        h[s] = fmaf(e, h[s], u);
                        if (OUT) acc = fmaf(c4[s][r], h[s], acc);
                    }
                    p[4 * q4 + r] = acc;
                }
            }
            if (OUT) {
                const float yv = row_transpose_sum(p, l16) + Dd * xrow[t16 + l16];
                sm.ys[(t16 + l16) * YS + cl] = yv;
            }
        }
        if (OUT) {
            __syncthreads();
            // y tile -> global: 16-byte pieces of 16 / sizeof(T) channels of one token
            constexpr int E = Io<T>::per16, PX = CB / E;
            T* yg = static_cast<T*>(a.y);
            for (int i = tid; i < TT * PX; i += 256) {
                const int r = i / PX, col = (i % PX) * E;
                if (r <= tl.last) {
                    T o[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) o[e] = from_f32<T>(sm.ys[r * YS + col + e]);
                    *reinterpret_cast<uint4*>(yg + (b * a.L + t0 + r) * a.Dc + c0 + col) =
                        *reinterpret_cast<const uint4*>(o);
                }
            }
        }
    }
    if (OUT) {
        if (seg == a.nseg - 1) {
#pragma unroll
            for (int s = 0; s < SPT; ++s) a.final_state[(b * a.Dc + c) * (int64_t)N + l16 + 16 * s] = h[s];
        }
    } else {
#pragma unroll
        for (int s = 0; s < SPT; ++s) a.seg_states[sidx + l16 + 16 * s] = h[s];
        if (l16 == 0) a.seg_sums[(b * (a.nseg - 1) + seg) * a.Dc + c] = dsum;
    }
}

// chain the segment end states in segment order; with no segments to chain it
// only writes the start state (h0 or zero) as the final state (empty sequence)
__global__ void __launch_bounds__(256) selective_carry_kernel(const float* A, const float* h0, float* seg_states,
                                                              const float* seg_sums, float* final_state, int64_t b,
                                                              int Dc, int N, int nseg) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= b * Dc * (int64_t)N) return;
    const int64_t bb = i / ((int64_t)Dc * N);
    const int c = (int)((i / N) % Dc), n = (int)(i % N);
    const float a2 = A[(int64_t)c * N + n] * kLog2e;
    float hv = h0 ? h0[i] : 0.0f;
    // eight segments' loads in flight per step of the chain
    constexpr int K = 8;
    for (int s0 = 0; s0 + 1 < nseg; s0 += K) {
        float loc[K], dec[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int s = s0 + k < nseg - 1 ? s0 + k : nseg - 2;
            loc[k] = seg_states[((bb * (nseg - 1) + s) * Dc + c) * (int64_t)N + n];
            dec[k] = seg_sums[(bb * (nseg - 1) + s) * Dc + c];
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (s0 + k < nseg - 1) {
                hv = fmaf(fast_exp2(a2 * dec[k]), hv, loc[k]);
                seg_states[((bb * (nseg - 1) + s0 + k) * Dc + c) * (int64_t)N + n] = hv;
            }
        }
    }
    if (final_state) final_state[i] = hv;
}

// ---------------------------------------------------------------------------
// dstate 16: one lane per channel, the whole state of the channel in its
// registers, so the sum over n stays in the lane.  One wavefront per
// workgroup (64 channels of one group); per tile the wavefront stages x and
// the step transposed to [channel][token] and the B, C rows to [token][n] in
// LDS (fp32), and every lane reads B and C rows as broadcasts.
//
// With the zero-order hold and no zero entry in A, the lane keeps g = A h:
//   g <- e g + (e - 1) B x = e (g + B x) - B x,   y = sum_n (C / A) g,
// three operations per entry and token for the update.  A wavefront whose
// channels have a zero entry of A keeps h and the (e - 1) / A factor with its
// limit delta.
// ---------------------------------------------------------------------------
constexpr int LN = 16;   // dstate of the lane kernel
constexpr int LCW = 64;  // channels per workgroup (one wavefront)

template <class T>
struct LaneCfg {
    static constexpr int TT = 16;                         // tokens per tile
    static constexpr int XS = TT + 4;                     // [channel][token] stride (conflict-free 16-byte reads)
    static constexpr int E = Io<T>::per16;
    static constexpr int KX = TT * LCW / E / 64;  // x (and step) pieces per lane
    static constexpr int NB = TT * LN / E;        // B (and C) pieces per tile
    static constexpr int KB = (NB + 63) / 64;
    static_assert(KX >= 1 && TT * LCW % (E * 64) == 0, "lane kernel tile split");
};

template <class T>
struct LaneLds {
    float xs[LCW * LaneCfg<T>::XS];
    float ds[LCW * LaneCfg<T>::XS];
    float bs[LaneCfg<T>::TT * LN];
    float cs[LaneCfg<T>::TT * LN];
};

template <class T>
struct LaneStage {
    uint4 x[LaneCfg<T>::KX], d[LaneCfg<T>::KX];
    uint4 b[LaneCfg<T>::KB], c[LaneCfg<T>::KB];
};

template <class T, bool OUT>
__device__ __forceinline__ void lane_load(LaneStage<T>& st, const Args& a, int64_t b, int64_t t0, int last, int c0,
                                          int g, int lane) {
    using CF = LaneCfg<T>;
    constexpr int PR = LCW / CF::E;  // pieces per x row
    const T* xg = static_cast<const T*>(a.x);
    const T* dg = static_cast<const T*>(a.delta);
#pragma unroll
    for (int k = 0; k < CF::KX; ++k) {
        const int i = lane + 64 * k, r = i / PR, col = (i % PR) * CF::E;
        const int64_t o = (b * a.L + t0 + (r <= last ? r : last)) * a.Dc + c0 + col;
        st.x[k] = *reinterpret_cast<const uint4*>(xg + o);
        st.d[k] = *reinterpret_cast<const uint4*>(dg + o);
    }
    constexpr int PB = LN / CF::E;
#pragma unroll
    for (int k = 0; k < CF::KB; ++k) {
        const int i = lane + 64 * k;
        if (i < CF::NB) {
            const int r = i / PB, col = (i % PB) * CF::E;
            const int64_t o = ((b * a.L + t0 + (r <= last ? r : last)) * a.G + g) * LN + col;
            st.b[k] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.B) + o);
            if (OUT) st.c[k] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.C) + o);
        }
    }
}

template <class T, bool OUT>
__device__ __forceinline__ void lane_store(LaneLds<T>& sm, const LaneStage<T>& st, const Args& a, int last, int c0,
                                           int lane) {
    using CF = LaneCfg<T>;
    constexpr int PR = LCW / CF::E;
#pragma unroll
    for (int k = 0; k < CF::KX; ++k) {
        const int i = lane + 64 * k, r = i / PR, col = (i % PR) * CF::E;
        const bool ok = r <= last;
        float v[CF::E], w[CF::E];
        Io<T>::unpack(st.x[k], v);
        Io<T>::unpack(st.d[k], w);
#pragma unroll
        for (int e = 0; e < CF::E; ++e) {
            float dec, inp;
            dt_front(a.fe, c0 + col + e, 0.0f, w[e], dec, inp);
            sm.xs[(col + e) * CF::XS + r] = ok ? v[e] : 0.0f;
            sm.ds[(col + e) * CF::XS + r] = ok ? dec : 0.0f;  // padding tokens: zero step
        }
    }
    constexpr int PB = LN / CF::E;
#pragma unroll
    for (int k = 0; k < CF::KB; ++k) {
        const int i = lane + 64 * k;
        if (i < CF::NB) {
            const int r = i / PB, col = (i % PB) * CF::E;
            const bool ok = r <= last;
            float v[CF::E];
            Io<T>::unpack(st.b[k], v);
#pragma unroll
            for (int e = 0; e < CF::E; ++e) sm.bs[r * LN + col + e] = ok ? v[e] : 0.0f;
            if (OUT) {
                Io<T>::unpack(st.c[k], v);
#pragma unroll
                for (int e = 0; e < CF::E; ++e) sm.cs[r * LN + col + e] = ok ? v[e] : 0.0f;
            }
        }
    }
}

// the token walk of one segment; GF: the state is kept as g = A h (zero-order hold, A has no zero)
template <class T, bool ZOH, bool OUT, bool GF>
__device__ __forceinline__ void lane_walk(LaneLds<T>& sm, const Args& a, float (&h)[LN], const float (&a2)[LN],
                                          const float (&ia)[LN], float& dsum, int64_t b,
                                          int64_t s0, int64_t s1, int c0, int g, int lane, float Dd) {
    using CF = LaneCfg<T>;
    constexpr int TT = CF::TT;
    const int c = c0 + lane;
    T* yg = static_cast<T*>(a.y);
    LaneStage<T> st;
    int last = (int)(s1 - s0 - 1 < TT - 1 ? s1 - s0 - 1 : TT - 1);
    lane_load<T, OUT>(st, a, b, s0, last, c0, g, lane);
    for (int64_t t0 = s0; t0 < s1; t0 += TT) {
        last = (int)(s1 - t0 - 1 < TT - 1 ? s1 - t0 - 1 : TT - 1);
        __syncthreads();
        lane_store<T, OUT>(sm, st, a, last, c0, lane);
        __syncthreads();
        if (t0 + TT < s1) {
            const int nl = (int)(s1 - t0 - TT - 1 < TT - 1 ? s1 - t0 - TT - 1 : TT - 1);
            lane_load<T, OUT>(st, a, b, t0 + TT, nl, c0, g, lane);
        }
#pragma unroll 1
        for (int t4 = 0; t4 < TT; t4 += 4) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.ds[lane * CF::XS + t4]);
            const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sm.xs[lane * CF::XS + t4]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t4 + r;
                const float dl = d4[r], xv = x4[r];
                if (!OUT) dsum += dl;
                float bv[LN], cv[LN];
#pragma unroll
                for (int q = 0; q < LN / 4; ++q) {
                    const f32x4 bq = *reinterpret_cast<const f32x4*>(&sm.bs[t * LN + 4 * q]);
                    bv[4 * q] = bq[0], bv[4 * q + 1] = bq[1], bv[4 * q + 2] = bq[2], bv[4 * q + 3] = bq[3];
                    if (OUT) {
                        const f32x4 cq = *reinterpret_cast<const f32x4*>(&sm.cs[t * LN + 4 * q]);
                        cv[4 * q] = cq[0], cv[4 * q + 1] = cq[1], cv[4 * q + 2] = cq[2], cv[4 * q + 3] = cq[3];
                    }
                }
                const float dx = dl * xv;
                float acc = 0.0f;
#pragma unroll
                for (int n = 0; n < LN; ++n) {
                    const float e = fast_exp2(dl * a2[n]);
                    if (GF) {
                        const float bx = bv[n] * xv;
                        h[n] = fmaf(e, h[n] + bx, -bx);
                        if (OUT) acc = fmaf(cv[n] * ia[n], h[n], acc);
                    } else {
                        float u;
                        if (ZOH) {
                            const float f = ia[n] != 0.0f ? fmaf(e, ia[n], -ia[n]) : dl;  // limit delta at A = 0
                            u = f * (bv[n] * xv);
                        } else {
                            u = dx * bv[n];
                        }
                        h[n] = fmaf(e, h[n], u);
                        if (OUT) acc = fmaf(cv[n], h[n], acc);
                    }
                }
                if (OUT && t <= last) yg[(b * a.L + t0 + t) * a.Dc + c] = from_f32<T>(fmaf(Dd, xv, acc));
            }
        }
    }
}

template <class T, bool ZOH, bool OUT>
__global__ void __launch_bounds__(64) selective_lane_kernel(Args a, uint32_t nitems) {
    __shared__ __align__(16) LaneLds<T> sm;
    const int nblk = a.Dc / LCW;
    const int nsegk = OUT ? a.nseg : a.nseg - 1;
    const uint32_t item = xcd_remap(blockIdx.x, nitems);
    const int cblk = (int)(item % (uint32_t)nblk);
    const int seg = (int)((item / (uint32_t)nblk) % (uint32_t)nsegk);
    const int64_t b = item / ((uint32_t)nblk * (uint32_t)nsegk);
    const int lane = threadIdx.x;
    const int c0 = cblk * LCW, c = c0 + lane;
    const int g = c0 / (a.Dc / a.G);
    const int64_t s0 = (int64_t)seg * a.Lseg;
    const int64_t s1 = s0 + a.Lseg < a.L ? s0 + a.Lseg : a.L;

    float a2[LN], ia[LN], h[LN];
    bool zero = false;
#pragma unroll
    for (int n = 0; n < LN; ++n) {
        const float Av = a.A[(int64_t)c * LN + n];
        a2[n] = Av * kLog2e;
        ia[n] = Av != 0.0f ? 1.0f / Av : 0.0f;
        zero |= Av == 0.0f;
    }
    const int64_t sidx = ((b * (a.nseg - 1) + seg) * a.Dc + c) * (int64_t)LN;
#pragma unroll
    for (int n = 0; n < LN; ++n) {
        float v = 0.0f;
        if (OUT) {
            if (seg == 0)
                v = a.h0 ? a.h0[(b * a.Dc + c) * (int64_t)LN + n] : 0.0f;
            else
                v = a.seg_states[sidx - (int64_t)a.Dc * LN + n];
        }
        h[n] = v;
    }
    const float Dd = (OUT && a.D) ? a.D[c] : 0.0f;
    float dsum = 0.0f;
    const bool gf = ZOH && !__any(zero);  // wavefront-uniform
    if (gf) {
#pragma unroll
        for (int n = 0; n < LN; ++n) h[n] *= a.A[(int64_t)c * LN + n];
        lane_walk<T, ZOH, OUT, ZOH>(sm, a, h, a2, ia, dsum, b, s0, s1, c0, g, lane, Dd);
#pragma unroll
        for (int n = 0; n < LN; ++n) h[n] *= ia[n];
    } else {
        lane_walk<T, ZOH, OUT, false>(sm, a, h, a2, ia, dsum, b, s0, s1, c0, g, lane, Dd);
    }
    if (OUT) {
        if (seg == a.nseg - 1) {
#pragma unroll
            for (int q = 0; q < LN / 4; ++q)
                *reinterpret_cast<f32x4*>(&a.final_state[(b * a.Dc + c) * (int64_t)LN + 4 * q]) =
                    f32x4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
        }
    } else {
#pragma unroll
        for (int q = 0; q < LN / 4; ++q)
            *reinterpret_cast<f32x4*>(&a.seg_states[sidx + 4 * q]) =
                f32x4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
        a.seg_sums[(b * (a.nseg - 1) + seg) * a.Dc + c] = dsum;
    }
}

template <class T, bool ZOH, bool OUT>
hipError_t launch_lane_pass(const Args& a, int64_t b, hipStream_t st) {
    const int nsegk = OUT ? a.nseg : a.nseg - 1;
    const uint32_t nitems = (uint32_t)(b * (a.Dc / LCW) * nsegk);
    if (nitems == 0) return hipSuccess;
    hipLaunchKernelGGL((selective_lane_kernel<T, ZOH, OUT>), dim3(nitems), dim3(64), 0, st, a, nitems);
    return hipGetLastError();
}

template <class T, int N, bool ZOH, bool OUT>
hipError_t launch_pass(const Args& a, int64_t b, hipStream_t st) {
    const int nsegk = OUT ? a.nseg : a.nseg - 1;
    const uint32_t nitems = (uint32_t)(b * (a.Dc / CB) * nsegk);
    if (nitems == 0) return hipSuccess;
    const size_t lds = sizeof(Lds<N>);
    hipLaunchKernelGGL((selective_scan_kernel<T, N, ZOH, OUT>), dim3(nitems), dim3(256), lds, st, a, nitems);
    return hipGetLastError();
}

template <class T, int N, bool ZOH>
hipError_t run(const Args& a, int64_t b, bool lane, hipStream_t st) {
    if (a.nseg > 1) {
        hipError_t e = lane ? launch_lane_pass<T, ZOH, false>(a, b, st) : launch_pass<T, N, ZOH, false>(a, b, st);
        if (e != hipSuccess) return e;
        const int64_t n = b * a.Dc * (int64_t)N;
        hipLaunchKernelGGL(selective_carry_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, a.A, a.h0,
                           a.seg_states, a.seg_sums, nullptr, b, a.Dc, N, a.nseg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return lane ? launch_lane_pass<T, ZOH, true>(a, b, st) : launch_pass<T, N, ZOH, true>(a, b, st);
}

template <class T, bool ZOH>
hipError_t by_n(const Args& a, int64_t b, int N, bool lane, hipStream_t st) {
    switch (N) {
        case 16: return run<T, 16, ZOH>(a, b, lane, st);
        case 32: return run<T, 32, ZOH>(a, b, false, st);
        case 48: return run<T, 48, ZOH>(a, b, false, st);
        case 64: return run<T, 64, ZOH>(a, b, false, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace sel

bool selective_supported(int64_t Dc, int64_t N, int64_t G) {
    return (N == 16 || N == 32 || N == 48 || N == 64) && G > 0 && Dc % G == 0 && (Dc / G) % sel::CB == 0;
}

// dstate 16 with 64 channels per group runs one lane per channel
static bool lane_kernel(int64_t Dc, int64_t N, int64_t G) { return N == sel::LN && (Dc / G) % sel::LCW == 0; }

SelectiveLayout selective_layout(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G, int64_t seg_len) {
    SelectiveLayout f{};
    int64_t Lseg;
    if (seg_len > 0) {
        Lseg = seg_len;
    } else {
        // segments enough for about eight wavefronts per SIMD (1024 SIMDs), none shorter than 256
        // tokens (one-lane-per-channel kernel) or 512 tokens (sixteen lanes per channel)
        const bool ln = lane_kernel(Dc, N, G);
        const int64_t waves = ln ? b * (Dc / sel::LCW) : b * (Dc / sel::CB) * 4;
        const int64_t target = ln ? 8192 : 4096, shortest = ln ? 256 : 512;
        int64_t nseg = 1;
        while (waves * nseg < target && L / (2 * nseg) >= shortest) nseg *= 2;
        Lseg = (L + nseg - 1) / nseg;
        Lseg = (Lseg + sel::TT - 1) / sel::TT * sel::TT;
    }
    if (Lseg <= 0) Lseg = sel::TT;
    f.seg_len = Lseg;
    f.nseg = L > 0 ? (int)((L + Lseg - 1) / Lseg) : 1;
    auto a256 = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t ns = (size_t)(f.nseg - 1);
    f.states = 0;
    f.sums = a256((size_t)(b * Dc * N) * ns * 4);
    f.total = f.nseg > 1 ? f.sums + a256((size_t)(b * Dc) * ns * 4) : 0;
    return f;
}

hipError_t launch_selective_scan(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G, int io, const DtFront& fe,
                                 const void* x, const void* delta, const float* A, const void* B, const void* C,
                                 const float* D, const float* h0, void* y, float* final_state, int64_t seg_len,
                                 void* workspace, hipStream_t st) {
    const SelectiveLayout f = selective_layout(b, L, Dc, N, G, seg_len);
    if (b == 0) return hipSuccess;
    if (L == 0) {  // the final state is the start state
        const int64_t n = b * Dc * N;
        hipLaunchKernelGGL(sel::selective_carry_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, A, h0,
                           nullptr, nullptr, final_state, b, (int)Dc, (int)N, 1);
        return hipGetLastError();
    }
    char* ws = static_cast<char*>(workspace);
    sel::Args a{x, delta, A, B, C, D, h0,
                f.nseg > 1 ? reinterpret_cast<float*>(ws + f.states) : nullptr,
                f.nseg > 1 ? reinterpret_cast<float*>(ws + f.sums) : nullptr,
                y, final_state, fe, L, f.seg_len, (int)Dc, (int)G, f.nseg};
    const bool zoh = fe.zoh != 0, lane = lane_kernel(Dc, N, G);
    if (io == 1)
        return zoh ? sel::by_n<bf16, true>(a, b, (int)N, lane, st) : sel::by_n<bf16, false>(a, b, (int)N, lane, st);
    return zoh ? sel::by_n<float, true>(a, b, (int)N, lane, st) : sel::by_n<float, false>(a, b, (int)N, lane, st);
}

}  // namespace ssd
