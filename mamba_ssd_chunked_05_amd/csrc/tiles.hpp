// tiles.hpp -- LDS tile helpers shared by the fast chunk kernels (fused.hip,
// wide.hip): headdim 64, 64-token sub-chunks, bf16 tiles in natural layout.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace fz {

constexpr int P = 64;
constexpr int QS = 64;        // tokens per chunk
constexpr int XS = P + 16;    // x row stride (bf16)

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int N>
struct Strides {
    static constexpr int BS = N + 16;  // B rows: transpose reads
    static constexpr int CS = N + 8;   // C rows: row reads
};

// Transpose read: rows [row0, row0+4) x columns [col0, col0+16) of a row-major
// bf16 LDS tile with leading dimension ld; lane (16g + j) receives column
// col0 + j, rows row0..row0+3 (row0 may differ between 16-lane groups).
__device__ __forceinline__ bf16x4 tr_read(const bf16* tile, int row0, int col0, int ld, int l16) {
    const bf16* p = tile + (row0 + (l16 >> 2)) * ld + col0 + 4 * (l16 & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 pack8(const bf16x4& a, const bf16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// four bf16 as floats, read from their packed halves (a shift or a mask each), so that a value rounded
// to bf16 in a pair is not rounded again on its own to recover it
__device__ __forceinline__ f32x4 bf16x4_to_f32(const bf16x4& h) {
    const uint2 u = __builtin_bit_cast(uint2, h);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}

__device__ __forceinline__ bf16x4 cvt4(const f32x4& v) {
    bf16x4 r;
    r[0] = static_cast<bf16>(v[0]);
    r[1] = static_cast<bf16>(v[1]);
    r[2] = static_cast<bf16>(v[2]);
    r[3] = static_cast<bf16>(v[3]);
    return r;
}

__device__ __forceinline__ uint4 ld16(const bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// Sub-chunk tiles are read through buffer resources: a resource starts at the tile's first element and
// its size ends with the last row inside the sequence (row_len elements of the last row), so the
// hardware's range check returns zero for rows past the end (whole 16-byte pieces: a row is in range
// entirely or not at all) and no load reaches past it.  Each load is then a wavefront-uniform resource
// plus one 32-bit per-thread byte offset, with no per-element select.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base, int64_t row_stride, int64_t rows,
                                                           int row_len) {
    const int64_t n = rows < QS ? rows : QS;
    const int bytes = n > 0 ? (int)(((n - 1) * row_stride + row_len) * 2) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ldbuf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// dt (fp32) and the cumulative log2 decay: over the chunk for the staged calls,
// restarting at every 64-token sub-chunk in the forward.  raw (the forward at dstate <= 128): no
// arrays -- the kernels read the step dt (b, L, H) bf16 themselves (rows of H elements), apply the
// front-end fe and A, and form each sub-chunk's cumulative decay in registers.
struct DtSrc {
    const float* dt_t;
    const float* cs;
    const bf16* raw = nullptr;
    const float* A = nullptr;
    DtFront fe{nullptr, 0, 0, 0, 0.0f, 0.0f};
    int H = 0;
};

}  // namespace fz
}  // namespace ssd
