// wgrad_reduce.hip -- finishes the split-K weight gradient: each output
// element is the sum of its `splits` fp32 partials taken in split order
// 0, 1, ..., splits-1, so the result does not depend on scheduling and is
// bit-identical from run to run (no value atomics anywhere).  A thread owns
// four consecutive elements (16-byte loads) and issues the loads of up to
// kBatch splits before adding them, in order (the layer shapes' 8 or 16
// splits in one round trip).
#include "gc_kernels.h"

namespace gc {
namespace {

constexpr int kBatch = 16;   // split loads in flight per thread

__device__ __forceinline__ void store4(float *p, const float4 &v) { __builtin_memcpy(p, &v, 16); }
__device__ __forceinline__ void store4(bf16_t *p, const float4 &v)
{
    const bf16_t h[4] = {from_f32<bf16_t>(v.x), from_f32<bf16_t>(v.y), from_f32<bf16_t>(v.z),
                         from_f32<bf16_t>(v.w)};
    __builtin_memcpy(p, h, 8);
}

template <typename T>
__global__ void __launch_bounds__(256) wgrad_reduce(const float *__restrict__ part,
                                                    T *__restrict__ dw, int splits, int n)
{
    // 16-byte loads need every split to start on a 16-byte boundary
    const int n4 = (n & 3) ? 0 : n >> 2;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(part) + i;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int z0 = 0; z0 < splits; z0 += kBatch) {
            float4 v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (z0 + j < splits) v[j] = src[size_t(z0 + j) * n4];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (z0 + j < splits) {
                    s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
                }
        }
        store4(dw + 4 * size_t(i), s);
    }
    // element by element when n is not a multiple of 4
    for (int i = 4 * n4 + blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int z = 0; z < splits; ++z) s += part[size_t(z) * n + i];
        dw[i] = from_f32<T>(s);
    }
}

// Rows of NP partial columns (NP a multiple of 4): the sum of each 16-byte
// group in split order as above, then each element to dw (column < N), db
// (column N) or nowhere (row padding).
template <typename T>
__global__ void __launch_bounds__(256) wgrad_reduce_bias(const float *__restrict__ part,
                                                         T *__restrict__ dw, T *__restrict__ db,
                                                         int splits, int OC, int N, int NP)
{
    const int n4 = OC * NP / 4;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(part) + i;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int z0 = 0; z0 < splits; z0 += kBatch) {
            float4 v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (z0 + j < splits) v[j] = src[size_t(z0 + j) * n4];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (z0 + j < splits) {
                    s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
                }
        }
        const int oc = 4 * i / NP, k0 = 4 * i - oc * NP;
        const float e[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = k0 + j;
            if (k < N) dw[size_t(oc) * N + k] = from_f32<T>(e[j]);
            else if (k == N) db[oc] = from_f32<T>(e[j]);
        }
    }
}

}  // namespace

template <typename T>
hipError_t launch_wgrad_reduce_bias(const float *part, void *dw, void *db, int splits, int OC, int N,
                                    int NP, hipStream_t s)
{
    if (reinterpret_cast<uintptr_t>(part) % 16 || NP % 4 || NP <= N) return hipErrorInvalidValue;
    int blocks = (OC * NP / 4 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(wgrad_reduce_bias<T>, dim3(blocks), dim3(256), 0, s, part, (T *)dw, (T *)db,
                       splits, OC, N, NP);
    return hipGetLastError();
}

template hipError_t launch_wgrad_reduce_bias<float>(const float *, void *, void *, int, int, int, int,
                                                    hipStream_t);
template hipError_t launch_wgrad_reduce_bias<bf16_t>(const float *, void *, void *, int, int, int, int,
                                                     hipStream_t);

template <typename T>
hipError_t launch_wgrad_reduce(const float *part, void *dw, int splits, int n, hipStream_t s)
{
    if (reinterpret_cast<uintptr_t>(part) % 16) return hipErrorInvalidValue;
    int blocks = ((n & 3 ? n : n / 4) + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(wgrad_reduce<T>, dim3(blocks), dim3(256), 0, s, part, (T *)dw, splits, n);
    return hipGetLastError();
}

template hipError_t launch_wgrad_reduce<float>(const float *, void *, int, int, hipStream_t);
template hipError_t launch_wgrad_reduce<bf16_t>(const float *, void *, int, int, hipStream_t);

}  // namespace gc
