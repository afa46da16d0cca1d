// calib.hip -- a measurement helper, not part of the SSD computation: a plain
// in-place read-modify-write stream over fp32 data, s <- a s + b.  It moves
// exactly the bytes of the decode step's state update (every element read once
// and written once) with none of its other work, so timed under the same
// conditions it gives the rate this chip achieves for that access pattern: the
// ceiling the decode step is compared with, next to the published HBM peak.
//
// Same streaming shape as the step kernel: 256-thread workgroups, two float4
// per thread with both loads issued before either store.
#include "../../include/ssd.h"
#include "../../include/ssd_bench.h"
#include "common.hpp"

namespace ssd {

__global__ void __launch_bounds__(256) rmw_stream_kernel(float4* __restrict__ s, int64_t n4, float a, float b) {
    const int64_t i0 = (int64_t)blockIdx.x * 512 + threadIdx.x, i1 = i0 + 256;
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
    if (i0 < n4) v0 = s[i0];
    if (i1 < n4) v1 = s[i1];
    v0.x = a * v0.x + b; v0.y = a * v0.y + b; v0.z = a * v0.z + b; v0.w = a * v0.w + b;
    v1.x = a * v1.x + b; v1.y = a * v1.y + b; v1.z = a * v1.z + b; v1.w = a * v1.w + b;
    if (i0 < n4) s[i0] = v0;
    if (i1 < n4) s[i1] = v1;
}

}  // namespace ssd

extern "C" ssd_status ssd_bench_rmw_stream(float* buf, size_t n, float a, float b, void* stream) {
    if (n == 0) return SSD_OK;
    if (!buf) return SSD_ERR_NULL;
    if (n % 4 || reinterpret_cast<uintptr_t>(buf) % 16) return SSD_ERR_UNSUPPORTED;
    const int64_t n4 = (int64_t)(n / 4);
    const int64_t grid = (n4 + 511) / 512;
    if (grid > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(ssd::rmw_stream_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<float4*>(buf), n4, a, b);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}
