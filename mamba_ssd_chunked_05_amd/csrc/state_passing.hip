// state_passing.hip -- chunk-order pass over the chunk states.
//
// Second half of the state kernel on the devotd.net cuTile Mamba-2 page
// (section 2): chunks are visited in order while the independent state
// elements run in parallel.  It rests on the associativity of the first-order
// recurrence ("3.3 Hardware-Aware algorithms ...", section 4.1): a whole chunk
// acts on the carried state as S -> 2^(l_end) S + local.
//
// Every thread owns four consecutive fp32 state elements of one (b, h) and
// walks the nC chunks, reading each chunk-local state once and writing the
// chunk-start state in its place.  Loads run eight chunks ahead of the
// dependent FMA chain so each wave keeps 8 x 1 KiB in flight; the pass is pure
// HBM streaming (one read and one write of the state tensor).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kSpDepth = 8;

__global__ void __launch_bounds__(256) state_passing_kernel(float* __restrict__ states, const float* __restrict__ cs,
                                                            const float* __restrict__ h0, float* __restrict__ fin,
                                                            int64_t nC, int H, int Q, int64_t PN) {
    const int64_t e4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e4 >= PN) return;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t bh = b * H + h;
    float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
    if (h0) S = *reinterpret_cast<const float4*>(h0 + bh * PN + e4);
    const int64_t cstride = (int64_t)H * PN;  // distance between consecutive chunks of one head
    float* base = states + (b * nC * H + h) * PN + e4;
    const float* lend = cs + bh * nC * Q + (Q - 1);
    for (int64_t c0 = 0; c0 < nC; c0 += kSpDepth) {
        float4 loc[kSpDepth];
        float dec[kSpDepth];
#pragma unroll
        for (int k = 0; k < kSpDepth; ++k) {
            if (c0 + k < nC) {
                loc[k] = *reinterpret_cast<const float4*>(base + (c0 + k) * cstride);
                dec[k] = fast_exp2(lend[(c0 + k) * Q]);
            }
        }
#pragma unroll
        for (int k = 0; k < kSpDepth; ++k) {
            if (c0 + k < nC) {
                *reinterpret_cast<float4*>(base + (c0 + k) * cstride) = S;
                S.x = dec[k] * S.x + loc[k].x;
                S.y = dec[k] * S.y + loc[k].y;
                S.z = dec[k] * S.z + loc[k].z;
                S.w = dec[k] * S.w + loc[k].w;
            }
        }
    }
    *reinterpret_cast<float4*>(fin + bh * PN + e4) = S;
}

hipError_t launch_state_passing(const Shape& s, float* states, const float* cs, const float* h0,
                                float* final_state, hipStream_t st) {
    const int64_t PN = s.P * s.N;
    if (s.b == 0) return hipSuccess;
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)s.H, (unsigned)s.b), block(256);
    hipLaunchKernelGGL(state_passing_kernel, grid, block, 0, st, states, cs, h0, final_state, s.nC, (int)s.H,
                       (int)(s.Q > 0 ? s.Q : 1), PN);
    return hipGetLastError();
}

}  // namespace ssd
