// step.hip -- O(1) single-token decode update, in place on the fixed-size state.
//
// The on-device state cache of "Compiler-First State Space Duality and
// Portable O(1) Autoregressive Caching for Inference" (Methodology: compiled
// on-device O(1) caching; the state never grows with the sequence):
//     S <- exp(dt A) S + dt x (outer) B,    y = C . S + D x   (after the update)
//
// Each workgroup streams a block of whole rows of one (b, h) state slice once:
// every thread reads float4s, updates them, writes them back and adds its share
// of C . S to the row sums.  Row sums are reduced with cross-lane shuffles
// when a row is a power-of-two number of float4s (one row never spans two
// wavefronts below N = 512), otherwise through LDS atomics.  The kernel is
// pure HBM streaming: 2 x 4 x P x N bytes of state per (b, h).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

// The state is read and written with non-temporal loads and stores: it is streamed once per step and
// not read again before the next step (measured cold on the decode state: 64 against 71 us per step;
// a plain read-modify-write stream of the same bytes gains the same way, 57 against 65 us).
typedef float ntf4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float4* p) {
    const ntf4 v = __builtin_nontemporal_load(reinterpret_cast<const ntf4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float4* p, float4 v) {
    const ntf4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<ntf4*>(p));
}


// Batch strides (in elements) sx of x and y, sdt of dt and sbc of B and C let
// the same kernel step one token of a (b, K, ...) multi-step layout.
//
// Workgroup i updates rows p0 .. p0 + RB - 1 of the state of (b, h) = i / nrb
// (nrb = P / RB row blocks per head): whole rows, so each row's C . S sum stays in
// the workgroup.  Each thread updates two float4 per pass with both loads issued
// before either update.
template <class T>
__global__ void __launch_bounds__(256) step_kernel(DtFront fe, float* __restrict__ state, const T* __restrict__ x,
                                                   const T* __restrict__ dt, const float* __restrict__ A,
                                                   const T* __restrict__ B, const T* __restrict__ C,
                                                   const float* __restrict__ D, T* __restrict__ y, int H, int P,
                                                   int N, int G, int RB, int64_t sx, int64_t sdt, int64_t sbc) {
    __shared__ float xs[256];
    __shared__ float ys[256];
    __shared__ float Bs[1024];
    __shared__ float Cs[1024];
    const int nrb = (P + RB - 1) / RB;
    const int64_t bh = blockIdx.x / nrb;
    const int p0 = (int)(blockIdx.x % nrb) * RB;
    const int rows = P - p0 < RB ? P - p0 : RB;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    for (int p = tid; p < rows; p += 256) {
        xs[p] = to_f32(x[b * sx + (int64_t)h * P + p0 + p]);
        ys[p] = 0.0f;
    }
    for (int n = tid; n < N; n += 256) {
        Bs[n] = to_f32(B[b * sbc + (int64_t)g * N + n]);
        Cs[n] = to_f32(C[b * sbc + (int64_t)g * N + n]);
    }
    float dec, d;  // decay and input steps
    dt_front(fe, h, A[h], to_f32(dt[b * sdt + h]), dec, d);
    const float a = fast_exp2(kLog2e * (dec * A[h]));
    __syncthreads();

    const int n4 = N / 4;
    const int64_t total4 = (int64_t)rows * n4;
    const bool pow2 = (n4 & (n4 - 1)) == 0;
    const int grp = n4 < 64 ? n4 : 64;  // lanes per reduction group
    float4* S = reinterpret_cast<float4*>(state + (bh * P + p0) * (int64_t)N);
    for (int64_t base = 0; base < total4; base += 512) {
        // two pieces per thread, loads first
        const int64_t i0 = base + tid, i1 = base + 256 + tid;
        const bool v0 = i0 < total4, v1 = i1 < total4;
        float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
        if (v0) s0 = ld_nt(&S[i0]);
        if (v1) s1 = ld_nt(&S[i1]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t idx = q ? i1 : i0;
            const bool valid = q ? v1 : v0;
            float4 sv = q ? s1 : s0;
            float part = 0.0f;
            int p = 0;
            if (valid) {
                p = (int)(idx / n4);
                const int n = (int)(idx % n4) * 4;
                const float u = d * xs[p];
                sv.x = a * sv.x + u * Bs[n + 0];
                sv.y = a * sv.y + u * Bs[n + 1];
                sv.z = a * sv.z + u * Bs[n + 2];
                sv.w = a * sv.w + u * Bs[n + 3];
                st_nt(&S[idx], sv);
                part = Cs[n + 0] * sv.x + Cs[n + 1] * sv.y + Cs[n + 2] * sv.z + Cs[n + 3] * sv.w;
            }
            if (pow2) {
                for (int off = grp >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
                if (valid && (lane & (grp - 1)) == 0) {
                    if (n4 <= 64)
                        ys[p] = part;
                    else
                        atomicAdd(&ys[p], part);
                }
            } else if (valid) {
                atomicAdd(&ys[p], part);
            }
        }
    }
    __syncthreads();
    const float Dh = D ? D[h] : 0.0f;
    for (int p = tid; p < rows; p += 256) y[b * sx + (int64_t)h * P + p0 + p] = from_f32<T>(ys[p] + Dh * xs[p]);
}

// four consecutive elements as floats (8- or 16-byte aligned)
__device__ __forceinline__ void load4(const bf16* p, float* f) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float* f) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x, f[1] = v.y, f[2] = v.z, f[3] = v.w;
}

constexpr int kStepK = 4;  // float4 of state per thread in step_lane_kernel

// Sum over each aligned group of N4 lanes, left in every lane of the group: lane swaps inside quads
// and rotations inside 16-lane rows (data-parallel moves, no trip through the LDS unit), then
// cross-lane shuffles between rows.
template <int N4>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N4 >= 4 && N4 <= 64 && (N4 & (N4 - 1)) == 0, "groups of 4 to 64 lanes");
    v = dpp_add<0xB1>(v);  // quad_perm [1, 0, 3, 2]: lane ^ 1
    v = dpp_add<0x4E>(v);  // quad_perm [2, 3, 0, 1]: lane ^ 2
    if (N4 == 8) v += __shfl_xor(v, 4, 64);
    if (N4 >= 16) {
        v = dpp_add<0x124>(v);  // row_ror 4
        v = dpp_add<0x128>(v);  // row_ror 8
    }
    if (N4 >= 32) v += __shfl_xor(v, 16, 64);
    if (N4 >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// The same update for dstate N = 4 N4 with N4 a power of two from 4 to 64 (dstate 16 to 256).
// Thread t owns the four state columns n = 4 (t % N4) .. + 3 of rows t / N4 + k (256 / N4), k < kStepK,
// of the block, so it needs only its own four values of B and of C and the x of its rows, loaded
// straight into registers; each row lies in N4 consecutive lanes of one wavefront, which reduce its
// C . S with cross-lane moves.  No LDS and no barrier.  The few small loads go out first and the state
// loads right after them, so the update of row k waits only for its own state piece (the load counter
// retires in issue order).
template <class T, int N4>
__global__ void __launch_bounds__(256) step_lane_kernel(DtFront fe, float* __restrict__ state,
                                                        const T* __restrict__ x, const T* __restrict__ dt,
                                                        const float* __restrict__ A, const T* __restrict__ B,
                                                        const T* __restrict__ C, const float* __restrict__ D,
                                                        T* __restrict__ y, int H, int P, int G, int RB, int64_t sx,
                                                        int64_t sdt, int64_t sbc) {
    constexpr int N = 4 * N4, R = 256 / N4;
    const int nrb = (P + RB - 1) / RB;
    const int64_t bh = blockIdx.x / nrb;
    const int p0 = (int)(blockIdx.x % nrb) * RB;
    const int rows = P - p0 < RB ? P - p0 : RB;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const int g = h / (H / G);
    const int tid = threadIdx.x, c4 = tid & (N4 - 1), r0 = tid / N4;
    // rows past the block read its last row instead (never stored): no branch holds the loads back
    int pr[kStepK];
#pragma unroll
    for (int k = 0; k < kStepK; ++k) pr[k] = r0 + k * R < rows ? r0 + k * R : rows - 1;
    float bq[4], cq[4], xv[kStepK];
    const float ah = A[h];
    const float dtv = to_f32(dt[b * sdt + h]);
    const float Dh = D ? D[h] : 0.0f;
    load4(B + b * sbc + (int64_t)g * N + 4 * c4, bq);
    load4(C + b * sbc + (int64_t)g * N + 4 * c4, cq);
    const T* xr = x + b * sx + (int64_t)h * P + p0;
#pragma unroll
    for (int k = 0; k < kStepK; ++k) xv[k] = to_f32(xr[pr[k]]);
    float4* S = reinterpret_cast<float4*>(state + (bh * P + p0) * (int64_t)N);
    float4 sv[kStepK];
#pragma unroll
    for (int k = 0; k < kStepK; ++k) sv[k] = ld_nt(&S[(int64_t)pr[k] * N4 + c4]);
    float dec, d;  // decay and input steps
    dt_front(fe, h, ah, dtv, dec, d);
    const float a = fast_exp2(kLog2e * (dec * ah));
    T* yr = y + b * sx + (int64_t)h * P + p0;
#pragma unroll
    for (int k = 0; k < kStepK; ++k) {
        const int p = r0 + k * R;
        if (p < rows) {  // the same for all N4 lanes of the row
            const float u = d * xv[k];
            float4 v = sv[k];
            v.x = a * v.x + u * bq[0];
            v.y = a * v.y + u * bq[1];
            v.z = a * v.z + u * bq[2];
            v.w = a * v.w + u * bq[3];
            st_nt(&S[(int64_t)p * N4 + c4], v);
            const float part = group_sum<N4>(cq[0] * v.x + cq[1] * v.y + cq[2] * v.z + cq[3] * v.w);
            if (c4 == 0) yr[p] = from_f32<T>(part + Dh * xv[k]);
        }
    }
}

static bool step_lane_ok(const Shape& s) {
    const int64_t n4 = s.N / 4;
    return s.N % 4 == 0 && n4 >= 4 && n4 <= 64 && (n4 & (n4 - 1)) == 0;
}

template <class T>
static void launch_step_lane(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt,
                             const float* A, const void* B, const void* C, const float* D, void* y, int RB,
                             int64_t nwg, int64_t sx, int64_t sdt, int64_t sbc, hipStream_t st) {
    const T *xt = (const T*)x, *dtt = (const T*)dt, *Bt = (const T*)B, *Ct = (const T*)C;
    T* yt = (T*)y;
    const dim3 grid((unsigned)nwg), block(256);
    const int H = (int)s.H, P = (int)s.P, G = (int)s.G;
    switch (s.N / 4) {
#define SSD_STEP_LANE(n4)                                                                                         \
    case n4:                                                                                                      \
        hipLaunchKernelGGL((step_lane_kernel<T, n4>), grid, block, 0, st, fe, state, xt, dtt, A, Bt, Ct, D, yt, H, \
                           P, G, RB, sx, sdt, sbc);                                                               \
        break;
        SSD_STEP_LANE(4)
        SSD_STEP_LANE(8)
        SSD_STEP_LANE(16)
        SSD_STEP_LANE(32)
        SSD_STEP_LANE(64)
#undef SSD_STEP_LANE
    }
}

// rows per workgroup: 1024 float4 of state (whole rows; at least one).  Measured on the decode
// state (64 x 80 heads, P 64, N 128), cold: 16 rows 72.2, 32 rows 70.4, 64 rows (one head) 71.8 us
// per step, against 65.2 us for a plain in-place read-modify-write of the same bytes.
static int step_rows(const Shape& s) {
    const int64_t rb = 4096 / s.N;
    return (int)(rb < 1 ? 1 : (rb > s.P ? s.P : rb));
}

// one decode token with batch strides sx (x, y), sdt (dt), sbc (B, C)
static hipError_t launch_step_strided(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt,
                                      const float* A, const void* B, const void* C, const float* D, void* y,
                                      int64_t sx, int64_t sdt, int64_t sbc, hipStream_t st) {
    const int64_t nbh = s.b * s.H;
    const int RB = step_rows(s);
    const int64_t nwg = nbh * ((s.P + RB - 1) / RB);
    if (step_lane_ok(s)) {
        if (s.io == 1)
            launch_step_lane<bf16>(s, fe, state, x, dt, A, B, C, D, y, RB, nwg, sx, sdt, sbc, st);
        else
            launch_step_lane<float>(s, fe, state, x, dt, A, B, C, D, y, RB, nwg, sx, sdt, sbc, st);
        return hipGetLastError();
    }
    if (s.io == 1)
        hipLaunchKernelGGL(step_kernel<bf16>, dim3((unsigned)nwg), dim3(256), 0, st, fe, state, (const bf16*)x,
                           (const bf16*)dt, A, (const bf16*)B, (const bf16*)C, D, (bf16*)y, (int)s.H, (int)s.P,
                           (int)s.N, (int)s.G, RB, sx, sdt, sbc);
    else
        hipLaunchKernelGGL(step_kernel<float>, dim3((unsigned)nwg), dim3(256), 0, st, fe, state, (const float*)x,
                           (const float*)dt, A, (const float*)B, (const float*)C, D, (float*)y, (int)s.H, (int)s.P,
                           (int)s.N, (int)s.G, RB, sx, sdt, sbc);
    return hipGetLastError();
}

hipError_t launch_step(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, void* y, hipStream_t st) {
    const int64_t nbh = s.b * s.H;
    if (nbh == 0) return hipSuccess;
    const int64_t sx = s.H * s.P, sdt = s.H, sbc = s.G * s.N;
    return launch_step_strided(s, fe, state, x, dt, A, B, C, D, y, sx, sdt, sbc, st);
}

// ---------------------------------------------------------------------------
// K decode steps over pre-staged inputs with the state held on chip
// ---------------------------------------------------------------------------
// The multi-step form of the same update (the on-device decode loop of the
// "Compiler-First State Space Duality ..." page, Methodology and Results: the
// state never leaves the device and no host round trip separates the steps).
// Inputs of all K steps are already on the device in the forward's layouts,
// x, y (b, K, H, P), dt (b, K, H), B, C (b, K, G, N); step k is token k.
//
// One workgroup per (b, h) holds the P x N fp32 state in registers for all K
// steps.  The 256 threads form a 16 x 16 grid over (row block, column block):
// thread t owns rows RT (t / 16) .. + RT - 1 and columns CT (t % 16) .. + CT - 1
// (RT = P / 16, CT = N / 16), so a step reads CT values of B and of C and RT of
// x from LDS for RT * CT state elements.  C . S is reduced over the 16 threads
// of a row block -- sixteen consecutive lanes -- with DPP moves.  Each block of
// KB steps stages x, dt, B, C in LDS (fp32) and leaves y in LDS, written out
// coalesced after the block.  The state crosses HBM once per call.
constexpr int kMultiKB = 16;  // steps per LDS block

// One block of KB steps' inputs in registers: x (KB x P), B and C (KB x N) as
// 16-byte pieces, thread t holding pieces t, t + 256, ...; loaded while the
// previous block is computed, then stored to LDS as fp32.
template <class T, int P, int N, int KB>
struct MultiBlock {
    static constexpr int V = 16 / sizeof(T);                 // elements per piece
    static constexpr int NX = (KB * P / V + 255) / 256;      // x pieces per thread
    static constexpr int NB = (KB * N / V + 255) / 256;      // B (and C) pieces per thread
    uint4 xv[NX], bv[NB], cv[NB];
    T draw;

    __device__ __forceinline__ void load(const T* __restrict__ x, const T* __restrict__ dt,
                                         const T* __restrict__ B, const T* __restrict__ C, int64_t b, int64_t K,
                                         int64_t k0, int kb, int h, int g, int H, int G, int tid) {
        // Rows past the block's kb steps load a valid row (the block's first) instead: the
        // step loop never reads them, and no select makes the loads wait here.
        const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int e = tid + 256 * i, r = e / (P / V), c = (e % (P / V)) * V;
            xv[i] = *reinterpret_cast<const uint4*>(x + (b * K + k0 + (r < kb ? r : 0)) * HP + (int64_t)h * P + c);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int e = tid + 256 * i, r = e / (N / V), c = (e % (N / V)) * V;
            const int64_t off = (b * K + k0 + (r < kb ? r : 0)) * GN + (int64_t)g * N + c;
            bv[i] = *reinterpret_cast<const uint4*>(B + off);
            cv[i] = *reinterpret_cast<const uint4*>(C + off);
        }
        draw = dt[(b * K + k0 + (tid < kb ? tid : 0)) * H + h];
        __builtin_amdgcn_sched_barrier(0);  // nothing that uses the pieces moves up to here
    }

    // 16 bytes -> V floats, on 32-bit words (bf16 is the upper half of an fp32)
    static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (V == 8) {
                f[2 * q] = __uint_as_float(w[q] << 16);
                f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
            } else {
                f[q] = __uint_as_float(w[q]);
            }
        }
    }

    __device__ __forceinline__ void store(float* xs, float* bs, float* cs, int tid) const {
        float f[V];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int e = tid + 256 * i;
            if (e < KB * P / V) {
                unpack(xv[i], f);
#pragma unroll
                for (int q = 0; q < V; q += 4)
                    *reinterpret_cast<float4*>(xs + e * V + q) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int e = tid + 256 * i;
            if (e < KB * N / V) {
                unpack(bv[i], f);
#pragma unroll
                for (int q = 0; q < V; q += 4)
                    *reinterpret_cast<float4*>(bs + e * V + q) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
                unpack(cv[i], f);
#pragma unroll
                for (int q = 0; q < V; q += 4)
                    *reinterpret_cast<float4*>(cs + e * V + q) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
            }
        }
    }
};

template <class T, int RT, int CT>
__global__ void __launch_bounds__(256) step_multi_kernel(DtFront fe, float* __restrict__ state, const T* __restrict__ x,
                                                         const T* __restrict__ dt, const float* __restrict__ A,
                                                         const T* __restrict__ B, const T* __restrict__ C,
                                                         const float* __restrict__ D, T* __restrict__ y, int64_t K,
                                                         int H, int G) {
    constexpr int P = 16 * RT, N = 16 * CT, KB = kMultiKB;
    __shared__ __align__(16) float xs[KB * P];
    __shared__ __align__(16) float bs[KB * N];
    __shared__ __align__(16) float cs[KB * N];
    __shared__ float ds[KB];
    __shared__ float as[KB];  // exp(dt A) of each step of the block
    __shared__ float ys[KB * P];
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const int g = h / (H / G);
    const int tid = threadIdx.x, cg = tid & 15, p0 = (tid >> 4) * RT, n0 = cg * CT;
    float s[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const float* row = state + (bh * P + p0 + i) * (int64_t)N + n0;
#pragma unroll
        for (int j = 0; j < CT; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + j);
            s[i][j] = v.x;
            s[i][j + 1] = v.y;
            s[i][j + 2] = v.z;
            s[i][j + 3] = v.w;
        }
    }
    const float al = A[h] * kLog2e;
    const float Dh = D ? D[h] : 0.0f;
    const int64_t HP = (int64_t)H * P;
    MultiBlock<T, P, N, KB> blk;
    blk.load(x, dt, B, C, b, K, 0, K < KB ? (int)K : KB, h, g, H, G, tid);
    for (int64_t k0 = 0; k0 < K; k0 += KB) {
        const int kb = K - k0 < KB ? (int)(K - k0) : KB;
        __syncthreads();  // the previous block's y is written out; the LDS block is free
        blk.store(xs, bs, cs, tid);
        if (tid < KB) {  // the step's decay and input step
            float dec, din;
            dt_front(fe, h, A[h], to_f32(blk.draw), dec, din);
            ds[tid] = din;
            as[tid] = fast_exp2(dec * al);
        }
        __syncthreads();
        if (k0 + KB < K) {  // the next block's inputs stream in while this one is computed
            const int64_t k1 = k0 + KB;
            blk.load(x, dt, B, C, b, K, k1, K - k1 < KB ? (int)(K - k1) : KB, h, g, H, G, tid);
        }
        // software pipeline: step kk + 1's B, C and x are read from LDS while step kk computes
        float bv[CT], cv[CT], xv[RT];
        auto fetch = [&](int kk, float* bq, float* cq, float* xq) {
#pragma unroll
            for (int j = 0; j < CT; j += 4) {
                const float4 b4 = *reinterpret_cast<const float4*>(bs + kk * N + n0 + j);
                const float4 c4 = *reinterpret_cast<const float4*>(cs + kk * N + n0 + j);
                bq[j] = b4.x, bq[j + 1] = b4.y, bq[j + 2] = b4.z, bq[j + 3] = b4.w;
                cq[j] = c4.x, cq[j + 1] = c4.y, cq[j + 2] = c4.z, cq[j + 3] = c4.w;
            }
#pragma unroll
            for (int i = 0; i < RT; ++i) xq[i] = xs[kk * P + p0 + i];
        };
        fetch(0, bv, cv, xv);
        for (int kk = 0; kk < kb; ++kk) {
            const float d = ds[kk];
            const float a = as[kk];
            float bn[CT], cn[CT], xn[RT];
            fetch(kk + 1 < kb ? kk + 1 : kk, bn, cn, xn);
            // all rows' partial sums first (two chains per row), then the row reductions, so the
            // independent chains interleave; lane cg of a row block keeps row p0 + cg
            float sum[RT];
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const float u = d * xv[i];
                float pa = 0.0f, pb = 0.0f;
#pragma unroll
                for (int j = 0; j < CT; j += 2) {
                    s[i][j] = a * s[i][j] + u * bv[j];
                    s[i][j + 1] = a * s[i][j + 1] + u * bv[j + 1];
                    pa += cv[j] * s[i][j];
                    pb += cv[j + 1] * s[i][j + 1];
                }
                sum[i] = pa + pb;
            }
#pragma unroll
            for (int i = 0; i < RT; ++i) sum[i] = row16_sum(sum[i]);
            float mine = sum[0], xm = xv[0];
#pragma unroll
            for (int i = 1; i < RT; ++i) {
                mine = cg == i ? sum[i] : mine;
                xm = cg == i ? xv[i] : xm;
            }
            if (cg < RT) ys[kk * P + p0 + cg] = mine + Dh * xm;
#pragma unroll
            for (int j = 0; j < CT; ++j) bv[j] = bn[j], cv[j] = cn[j];
#pragma unroll
            for (int i = 0; i < RT; ++i) xv[i] = xn[i];
        }
        __syncthreads();
        for (int e = tid; e < kb * P; e += 256) {
            const int kk = e / P, pp = e % P;
            y[(b * K + k0 + kk) * HP + (int64_t)h * P + pp] = from_f32<T>(ys[e]);
        }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        float* row = state + (bh * P + p0 + i) * (int64_t)N + n0;
#pragma unroll
        for (int j = 0; j < CT; j += 4)
            *reinterpret_cast<float4*>(row + j) = make_float4(s[i][j], s[i][j + 1], s[i][j + 2], s[i][j + 3]);
    }
}

// static LDS of one block of steps (x, y: KB x P; B, C: KB x N; fp32) within 64 KiB,
// and at most 64 state elements per thread
constexpr bool multi_ok(int RT, int CT) {
    return RT * CT <= 64 && 4 * kMultiKB * (2 * 16 * RT + 2 * 16 * CT) + 64 <= 65536;
}

template <class T, int RT, int CT>
static hipError_t launch_multi(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt, const float* A,
                               const void* B, const void* C, const float* D, void* y, hipStream_t st) {
    if constexpr (multi_ok(RT, CT)) {
        hipLaunchKernelGGL((step_multi_kernel<T, RT, CT>), dim3((unsigned)(s.b * s.H)), dim3(256), 0, st, fe, state,
                           (const T*)x, (const T*)dt, A, (const T*)B, (const T*)C, D, (T*)y, s.L, (int)s.H,
                           (int)s.G);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <class T, int CT>
static hipError_t multi_by_rt(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt, const float* A,
                              const void* B, const void* C, const float* D, void* y, hipStream_t st) {
    switch (s.P / 16) {
#define SSD_RT(r) \
    case r: return launch_multi<T, r, CT>(s, fe, state, x, dt, A, B, C, D, y, st);
        SSD_RT(1) SSD_RT(2) SSD_RT(3) SSD_RT(4) SSD_RT(5) SSD_RT(6) SSD_RT(7) SSD_RT(8)
        SSD_RT(9) SSD_RT(10) SSD_RT(11) SSD_RT(12) SSD_RT(13) SSD_RT(14) SSD_RT(15) SSD_RT(16)
#undef SSD_RT
    }
    return hipErrorInvalidValue;
}

template <class T>
static hipError_t multi_by_ct(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt, const float* A,
                              const void* B, const void* C, const float* D, void* y, hipStream_t st) {
    switch (s.N / 16) {
        case 4: return multi_by_rt<T, 4>(s, fe, state, x, dt, A, B, C, D, y, st);
        case 8: return multi_by_rt<T, 8>(s, fe, state, x, dt, A, B, C, D, y, st);
        case 16: return multi_by_rt<T, 16>(s, fe, state, x, dt, A, B, C, D, y, st);
        case 32: return multi_by_rt<T, 32>(s, fe, state, x, dt, A, B, C, D, y, st);
        case 64: return multi_by_rt<T, 64>(s, fe, state, x, dt, A, B, C, D, y, st);
    }
    return hipErrorInvalidValue;
}

bool step_multi_on_chip(const Shape& s) {
    const int rt = (int)(s.P / 16), ct = (int)(s.N / 16);
    const bool ct_ok = ct == 4 || ct == 8 || ct == 16 || ct == 32 || ct == 64;
    return s.P % 16 == 0 && s.N % 16 == 0 && rt >= 1 && rt <= 16 && ct_ok && multi_ok(rt, ct);
}

hipError_t launch_step_multi(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt, const float* A,
                             const void* B, const void* C, const float* D, void* y, hipStream_t st) {
    const int64_t nbh = s.b * s.H;
    if (nbh == 0 || s.L == 0) return hipSuccess;
    if (step_multi_on_chip(s))
        return s.io == 1 ? multi_by_ct<bf16>(s, fe, state, x, dt, A, B, C, D, y, st)
                         : multi_by_ct<float>(s, fe, state, x, dt, A, B, C, D, y, st);
    // other state shapes: one single-step launch per token, still without a host round trip
    const size_t e = s.io == 1 ? 2 : 4;
    const int64_t sx = s.L * s.H * s.P, sdt = s.L * s.H, sbc = s.L * s.G * s.N;
    for (int64_t k = 0; k < s.L; ++k) {
        const char* xk = static_cast<const char*>(x) + k * s.H * s.P * e;
        const char* dk = static_cast<const char*>(dt) + k * s.H * e;
        const char* bk = static_cast<const char*>(B) + k * s.G * s.N * e;
        const char* ck = static_cast<const char*>(C) + k * s.G * s.N * e;
        char* yk = static_cast<char*>(y) + k * s.H * s.P * e;
        const hipError_t err0 = launch_step_strided(s, fe, state, xk, dk, A, bk, ck, D, yk, sx, sdt, sbc, st);
        if (err0 != hipSuccess) return err0;
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace ssd
