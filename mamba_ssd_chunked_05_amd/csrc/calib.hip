// calib.hip -- a measurement helper, not part of the SSD computation: a plain
// in-place read-modify-write stream over fp32 data, s <- a s + b.  It moves
// exactly the bytes of the decode step's state update (every element read once
// and written once) with none of its other work, so timed under the same
// conditions it gives the rate this chip achieves for that access pattern: the
// ceiling the decode step is compared with, next to the published HBM peak.
//
// 256-thread workgroups, two float4 per thread with both loads issued before
// either store, non-temporal loads and stores (data streamed once, as in the
// step): the fastest of the plain streaming forms measured cold on the decode
// state's 168 MB (57 us against 65 us with ordinary loads and stores).
#include "../../include/ssd.h"
#include "../../include/ssd_bench.h"
#include "common.hpp"

namespace ssd {

typedef float nt4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ nt4f ld_stream(const float4* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const nt4f*>(p));
}
__device__ __forceinline__ void st_stream(float4* p, nt4f v) {
    __builtin_nontemporal_store(v, reinterpret_cast<nt4f*>(p));
}

__global__ void __launch_bounds__(256) rmw_stream_kernel(float4* __restrict__ s, int64_t n4, float a, float b) {
    const int64_t i0 = (int64_t)blockIdx.x * 512 + threadIdx.x, i1 = i0 + 256;
    nt4f v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
    if (i0 < n4) v0 = ld_stream(&s[i0]);
    if (i1 < n4) v1 = ld_stream(&s[i1]);
    v0 = a * v0 + b;
    v1 = a * v1 + b;
    if (i0 < n4) st_stream(&s[i0], v0);
    if (i1 < n4) st_stream(&s[i1], v1);
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
