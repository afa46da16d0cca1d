// common.hpp -- device helpers shared by the libssd kernels (gfx950 only).
//
// MFMA fragment conventions used throughout (verified lane layouts of
// v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32):
//   A operand (16 x K):  lane l holds row (l % 16) and 8 K-positions;
//   B operand (K x 16):  lane l holds column (l % 16) and the same 8 K-positions;
//   accumulator (16x16): lane l holds rows 4*(l/16) + r, r = 0..3, column l % 16.
// Only the pairing of K-positions between A and B matters for a product, so
// each kernel picks whichever K-order is cheapest to load, as long as both
// operands use the same one ("frag slot s of lane-group g <-> k(g, s)").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <class T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }  // RNE

// hardware 2^x (v_exp_f32); exact limits: 2^-inf = 0, large negative -> 0
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// The dt front-end for head h with decay rate a_h: the decay step dec and the
// input step inp from the raw value.  softplus(d) = log(1 + e^d), evaluated as
// d + log1p(e^-d) for d > 0; the zero-order-hold input step is expm1(d a) / a.
template <class FE>
__device__ __forceinline__ void dt_front(const FE& fe, int h, float a_h, float raw, float& dec, float& inp) {
    float d = raw;
    if (fe.bias) d += fe.bias[h];
    if (fe.softplus) d = d > 0.0f ? d + log1pf(expf(-d)) : log1pf(expf(d));
    if (fe.clamp) d = fminf(fmaxf(d, fe.lo), fe.hi);
    dec = d;
    inp = fe.zoh && a_h != 0.0f ? expm1f(d * a_h) / a_h : d;
}

// ---------------------------------------------------------------------------
// MFMA fragments: 8 operand values per lane
// ---------------------------------------------------------------------------
template <class T>
struct Frag;

template <>
struct Frag<bf16> {
    bf16x8 v;
};

template <>
struct Frag<float> {
    float v[8];
};

// acc += A * B over the 32 K-positions carried by the two fragments.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

// fp32 operands: slot s of every lane-group forms one 16x16x4 product.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

template <class T>
__device__ __forceinline__ void frag_set(Frag<T>& f, int s, float v);
template <>
__device__ __forceinline__ void frag_set<bf16>(Frag<bf16>& f, int s, float v) { f.v[s] = static_cast<bf16>(v); }
template <>
__device__ __forceinline__ void frag_set<float>(Frag<float>& f, int s, float v) { f.v[s] = v; }

template <class T>
__device__ __forceinline__ void frag_zero(Frag<T>& f) {
#pragma unroll
    for (int s = 0; s < 8; ++s) frag_set<T>(f, s, 0.0f);
}

// 8 consecutive elements from LDS (16-byte aligned for bf16, 32-byte for fp32)
template <class T>
__device__ __forceinline__ void frag_load8(Frag<T>& f, const T* p);
template <>
__device__ __forceinline__ void frag_load8<bf16>(Frag<bf16>& f, const bf16* p) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ void frag_load8<float>(Frag<float>& f, const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// two runs of 4 consecutive elements: slots 0..3 from p0, 4..7 from p1
template <class T>
__device__ __forceinline__ void frag_load4x2(Frag<T>& f, const T* p0, const T* p1);
template <>
__device__ __forceinline__ void frag_load4x2<bf16>(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <>
__device__ __forceinline__ void frag_load4x2<float>(Frag<float>& f, const float* p0, const float* p1) {
    float4 a = *reinterpret_cast<const float4*>(p0);
    float4 b = *reinterpret_cast<const float4*>(p1);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// ---------------------------------------------------------------------------
// global loads of 8 consecutive io elements as floats
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8_f32(const float* p, float out[8]) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void load8_f32(const bf16* p, float out[8]) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = static_cast<float>(v[i]);
}

// ---------------------------------------------------------------------------
// cross-lane sums with data-parallel moves (no trip through the LDS unit)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// the sum over each row of 16 lanes, left in every lane of the row: lane swaps inside quads
// (quad_perm [1,0,3,2] and [2,3,0,1]), then rotations by 4 and 8 inside the row
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    v = dpp_add<0x124>(v);
    return dpp_add<0x128>(v);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Four row sums at once: lane l16 of each row of 16 ends with the sum over the row of v[l16 / 4].  Each
// exchange halves the values a lane keeps: with lane l16 ^ 8 (rotation by 8 inside the row) it keeps
// v[2 b3 + 0, 1], with the mirrored lane of its half row (7 - l16 % 8, the opposite bit 2) it keeps
// v[2 b3 + b2] (b3, b2: bits 3 and 2 of l16); the quad then holds four partial sums of the same value.
__device__ __forceinline__ float row16_sum4(float v0, float v1, float v2, float v3, int l16) {
    const bool b3 = (l16 & 8) != 0, b2 = (l16 & 4) != 0;
    float k0 = b3 ? v2 : v0, k1 = b3 ? v3 : v1;
    k0 += dpp_mov<0x128>(b3 ? v0 : v2);
    k1 += dpp_mov<0x128>(b3 ? v1 : v3);
    float m = b2 ? k1 : k0;
    m += dpp_mov<0x141>(b2 ? k0 : k1);
    m = dpp_add<0xB1>(m);
    return dpp_add<0x4E>(m);
}

// inclusive prefix sum over the 64 lanes of a wavefront with data-parallel moves: shifts by 1, 2, 4 and
// 8 lanes inside each row of 16 (a lane with no source adds zero), then each row's last value added to
// the rows after it (row broadcasts of lanes 15 and 31)
// the value lane `src` (a constant) holds, in a scalar register: a lane read, no LDS permute; every lane of
// the wavefront must hold a valid value there
__device__ __forceinline__ float lane_read(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
// the value the first lane of this lane's 16-lane row holds
__device__ __forceinline__ float row_first(float v, int lane) {
    const float r0 = lane_read(v, 0), r1 = lane_read(v, 16), r2 = lane_read(v, 32), r3 = lane_read(v, 48);
    const int g = lane >> 4;
    return g < 2 ? (g == 0 ? r0 : r1) : (g == 2 ? r2 : r3);
}

__device__ __forceinline__ float wave_incl_scan(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

// ---------------------------------------------------------------------------
// workgroup -> XCD-contiguous work mapping.  Workgroups are dispatched
// round-robin over the 8 XCDs (id % 8); this bijection gives every XCD a
// contiguous range of logical work items so that neighbours (e.g. the heads
// of one chunk, which share B and C) share one L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
    const uint32_t nx = 8;
    uint32_t q = n / nx, rem = n % nx;
    uint32_t x = id % nx, k = id / nx;
    return x * q + (x < rem ? x : rem) + k;
}

// The same XCD ranges walked from their end.  An output kernel that follows a chunk-state kernel over the
// same items starts with the items that kernel ran last, whose x and B rows are then the most likely to
// still sit in the memory-side cache.
__device__ __forceinline__ uint32_t xcd_remap_rev(uint32_t id, uint32_t n) {
    const uint32_t nx = 8;
    uint32_t q = n / nx, rem = n % nx;
    uint32_t x = id % nx, k = id / nx;
    const uint32_t cnt = q + (x < rem ? 1u : 0u);  // items of XCD x
    return x * q + (x < rem ? x : rem) + (cnt - 1u - k);
}

}  // namespace ssd
