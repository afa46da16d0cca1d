// chunk_cumsum.hip -- in-chunk cumulative sum of dt*A in log2 units.
//
// Follows the first kernel of the devotd.net page on the NVIDIA / Jane Street
// cuTile Mamba-2 forward kernels (section 2 and its listing): load a chunk of
// dt with zero padding past the sequence end, upcast to fp32, multiply by the
// head's A, cumulative-sum along the chunk and scale by log2(e).  The output
// layout is (b, H, nC, Q) so the later stages read each chunk's values as one
// contiguous run (the layout change of that page's section 3).
//
// One wavefront per (b, h, c), walking the chunk in blocks of 512 positions:
// each lane owns up to 8 consecutive positions of a block and sums them
// serially, a 6-step wavefront prefix over the lane totals gives every lane its
// offset, and the block total carries into the next block.  Bandwidth-trivial.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

template <class T>
__global__ void __launch_bounds__(256) chunk_cumsum_kernel(DtFront fe, const T* __restrict__ dt,
                                                           const float* __restrict__ A, float* __restrict__ dt_t,
                                                           float* __restrict__ cs, int64_t L, int H, int Q, int64_t nC,
                                                           int64_t nwaves) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= nwaves) return;
    const int h = (int)(wid % H);
    const int64_t c = (wid / H) % nC;
    const int64_t b = wid / ((int64_t)H * nC);
    const float a = A[h];
    const int64_t base = ((b * H + h) * nC + c) * Q;
    float carry = 0.0f;  // sum over the chunk's earlier 512-token blocks
    for (int q0 = 0; q0 < Q; q0 += 512) {
        const int qb = Q - q0 < 512 ? Q - q0 : 512;
        const int E = (qb + 63) / 64;  // positions per lane in this block (<= 8)
        float v[8], d[8];  // cumulative decay, input step
        float run = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = 0.0f;
            d[e] = 0.0f;
            if (e < E) {
                const int i = lane * E + e;
                const int64_t t = c * Q + q0 + i;
                float dec = 0.0f;
                if (i < qb && t < L) dt_front(fe, h, a, to_f32(dt[(b * L + t) * H + h]), dec, d[e]);
                run += dec * a;
                v[e] = run;
            }
        }
        // inclusive prefix of the lane totals across the wavefront
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(incl, off, 64);
            if (lane >= off) incl += up;
        }
        float excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.0f;
        excl += carry;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = lane * E + e;
            if (e < E && i < qb) {
                cs[base + q0 + i] = (excl + v[e]) * kLog2e;
                dt_t[base + q0 + i] = d[e];
            }
        }
        carry += __shfl(incl, 63, 64);
    }
}

hipError_t launch_chunk_cumsum(const Shape& s, const DtFront& fe, const void* dt, const float* A, float* dt_t,
                               float* cs, hipStream_t st) {
    const int64_t nwaves = s.b * s.H * s.nC;
    if (nwaves == 0) return hipSuccess;
    dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
    if (s.io == 1)
        hipLaunchKernelGGL(chunk_cumsum_kernel<bf16>, grid, block, 0, st, fe, (const bf16*)dt, A, dt_t, cs, s.L,
                           (int)s.H, (int)s.Q, s.nC, nwaves);
    else
        hipLaunchKernelGGL(chunk_cumsum_kernel<float>, grid, block, 0, st, fe, (const float*)dt, A, dt_t, cs, s.L,
                           (int)s.H, (int)s.Q, s.nC, nwaves);
    return hipGetLastError();
}

}  // namespace ssd
