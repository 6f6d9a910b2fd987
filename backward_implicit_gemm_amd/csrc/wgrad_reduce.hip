// wgrad_reduce.hip -- finishes the split-K weight gradient: each output
// element is the sum of its `splits` fp32 partials taken in split order
// 0, 1, ..., splits-1, so the result does not depend on scheduling and is
// bit-identical from run to run (no value atomics anywhere).
#include "gc_kernels.h"

namespace gc {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) wgrad_reduce(const float *__restrict__ part,
                                                    T *__restrict__ dw, int splits, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int z = 0; z < splits; ++z) s += part[size_t(z) * n + i];
        dw[i] = from_f32<T>(s);
    }
}

}  // namespace

template <typename T>
hipError_t launch_wgrad_reduce(const float *part, void *dw, int splits, int n, hipStream_t s)
{
    int blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(wgrad_reduce<T>, dim3(blocks), dim3(256), 0, s, part, (T *)dw, splits, n);
    return hipGetLastError();
}

template hipError_t launch_wgrad_reduce<float>(const float *, void *, int, int, hipStream_t);
template hipError_t launch_wgrad_reduce<bf16_t>(const float *, void *, int, int, hipStream_t);

}  // namespace gc
