// step.hip -- O(1) single-token decode update, in place on the fixed-size state.
//
// The on-device state cache of "Compiler-First State Space Duality and
// Portable O(1) Autoregressive Caching for Inference" (Methodology: compiled
// on-device O(1) caching; the state never grows with the sequence):
//     S <- exp(dt A) S + dt x (outer) B,    y = C . S + D x   (after the update)
//
// One workgroup per (b, h).  The P x N fp32 state slice is streamed once:
// every thread reads a float4, updates it, writes it back and adds its share
// of C . S to the row sum.  Row sums are reduced with cross-lane shuffles
// when a row is a power-of-two number of float4s (one row never spans two
// wavefronts below N = 512), otherwise through LDS atomics.  The kernel is
// pure HBM streaming: 2 x 4 x P x N bytes of state per (b, h).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

template <class T>
__global__ void __launch_bounds__(256) step_kernel(float* __restrict__ state, const T* __restrict__ x,
                                                   const T* __restrict__ dt, const float* __restrict__ A,
                                                   const T* __restrict__ B, const T* __restrict__ C,
                                                   const float* __restrict__ D, T* __restrict__ y, int H, int P,
                                                   int N, int G) {
    __shared__ float xs[256];
    __shared__ float ys[256];
    __shared__ float Bs[1024];
    __shared__ float Cs[1024];
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    for (int p = tid; p < P; p += 256) {
        xs[p] = to_f32(x[bh * P + p]);
        ys[p] = 0.0f;
    }
    for (int n = tid; n < N; n += 256) {
        Bs[n] = to_f32(B[(b * G + g) * N + n]);
        Cs[n] = to_f32(C[(b * G + g) * N + n]);
    }
    const float d = to_f32(dt[bh]);
    const float a = fast_exp2(kLog2e * (d * A[h]));
    __syncthreads();

    const int n4 = N / 4;
    const int64_t total4 = (int64_t)P * n4;
    const bool pow2 = (n4 & (n4 - 1)) == 0;
    const int grp = n4 < 64 ? n4 : 64;  // lanes per reduction group
    float4* S = reinterpret_cast<float4*>(state + bh * (int64_t)P * N);
    for (int64_t base = 0; base < total4; base += 256) {
        const int64_t idx = base + tid;
        const bool valid = idx < total4;
        float part = 0.0f;
        int p = 0;
        if (valid) {
            p = (int)(idx / n4);
            const int n = (int)(idx % n4) * 4;
            float4 s = S[idx];
            const float u = d * xs[p];
            s.x = a * s.x + u * Bs[n + 0];
            s.y = a * s.y + u * Bs[n + 1];
            s.z = a * s.z + u * Bs[n + 2];
            s.w = a * s.w + u * Bs[n + 3];
            S[idx] = s;
            part = Cs[n + 0] * s.x + Cs[n + 1] * s.y + Cs[n + 2] * s.z + Cs[n + 3] * s.w;
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
    __syncthreads();
    const float Dh = D ? D[h] : 0.0f;
    for (int p = tid; p < P; p += 256) y[bh * P + p] = from_f32<T>(ys[p] + Dh * xs[p]);
}

hipError_t launch_step(const Shape& s, float* state, const void* x, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, void* y, hipStream_t st) {
    const int64_t nbh = s.b * s.H;
    if (nbh == 0) return hipSuccess;
    if (s.io == 1)
        hipLaunchKernelGGL(step_kernel<bf16>, dim3((unsigned)nbh), dim3(256), 0, st, state, (const bf16*)x,
                           (const bf16*)dt, A, (const bf16*)B, (const bf16*)C, D, (bf16*)y, (int)s.H, (int)s.P,
                           (int)s.N, (int)s.G);
    else
        hipLaunchKernelGGL(step_kernel<float>, dim3((unsigned)nbh), dim3(256), 0, st, state, (const float*)x,
                           (const float*)dt, A, (const float*)B, (const float*)C, D, (float*)y, (int)s.H, (int)s.P,
                           (int)s.N, (int)s.G);
    return hipGetLastError();
}

}  // namespace ssd
