// tiles.hpp -- LDS tile helpers shared by the fast chunk kernels (fused.hip,
// wide.hip): headdim 64, 64-token sub-chunks, bf16 tiles in natural layout.
#pragma once

#include "common.hpp"

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

__device__ __forceinline__ bf16x4 cvt4(const f32x4& v) {
    bf16x4 r;
    r[0] = static_cast<bf16>(v[0]);
    r[1] = static_cast<bf16>(v[1]);
    r[2] = static_cast<bf16>(v[2]);
    r[3] = static_cast<bf16>(v[3]);
    return r;
}

__device__ __forceinline__ uint4 ld16(const bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// dt (fp32) and the cumulative log2 decay: over the chunk for the staged calls,
// restarting at every 64-token sub-chunk in the forward.
struct DtSrc {
    const float* dt_t;
    const float* cs;
};

}  // namespace fz
}  // namespace ssd
