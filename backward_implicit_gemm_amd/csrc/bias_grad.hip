// bias_grad.hip -- bias gradient of the convolution layer:
//     db[oc] = sum over (b, oh, ow) of dz[b][oc][oh][ow],  dz = dy * (y > 0)
// (dy without a ReLU).  Two fixed-order stages, so the result is
// bit-reproducible:
//   1. workgroup c sums images [c*IPC, (c+1)*IPC): their IPC*OC*P values
//      are contiguous, so the workgroup reads them with consecutive threads on
//      consecutive elements, masks them and stages them in LDS; then thread
//      oc sums its channel's P values of each image, in (image, position)
//      order, and writes one fp32 partial per (c, oc).  (When the chunk does
//      not fit the LDS budget, thread oc reads its values from global memory
//      directly, in the same order, so the result does not depend on which
//      form runs);
//   2. one workgroup per channel sums the partials over c: thread t takes
//      c = t, t+256, ... in order, then a fixed tree in LDS combines the 256
//      thread sums; the result is rounded once to the storage type.
#include "gc_kernels.h"

namespace gc {
namespace {

constexpr int kIPC = 4;          // images per workgroup of stage 1
constexpr int kStageMax = 12288; // values (fp32, 48 KB of LDS) a stage-1 chunk may stage

template <typename T, bool STAGED>
__global__ void __launch_bounds__(256) bias_partials(const T *__restrict__ dy,
                                                     const T *__restrict__ ym,
                                                     float *__restrict__ part, Geom g, int relu)
{
    extern __shared__ float dzs[];   // STAGED: the chunk's masked dz, [img][oc][p]
    const int c = blockIdx.x;
    const int b0 = c * kIPC, nb = min(kIPC, g.B - b0);
    const size_t base = size_t(b0) * g.OC * g.P;
    if (STAGED) {
        const int n = nb * g.OC * g.P;
        for (int e = threadIdx.x; e < n; e += blockDim.x) {
            float v = to_f32(dy[base + e]);
            if (relu && !(to_f32(ym[base + e]) > 0.f)) v = 0.f;
            dzs[e] = v;
        }
        __syncthreads();
    }
    for (int oc = threadIdx.x; oc < g.OC; oc += blockDim.x) {
        float s = 0.f;
        for (int i = 0; i < nb; ++i) {
            const int row = (i * g.OC + oc) * g.P;
            for (int p = 0; p < g.P; ++p) {
                float v;
                if (STAGED) {
                    v = dzs[row + p];
                } else {
                    v = to_f32(dy[base + row + p]);
                    if (relu && !(to_f32(ym[base + row + p]) > 0.f)) v = 0.f;
                }
                s += v;
            }
        }
        part[size_t(c) * g.OC + oc] = s;
    }
}

template <typename T>
__global__ void __launch_bounds__(256) bias_final(const float *__restrict__ part, T *__restrict__ db,
                                                  int chunks, int OC)
{
    __shared__ float red[256];
    const int oc = blockIdx.x, t = threadIdx.x;
    float s = 0.f;
    for (int c = t; c < chunks; c += 256) s += part[size_t(c) * OC + oc];
    red[t] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) red[t] += red[t + w];
        __syncthreads();
    }
    if (t == 0) db[oc] = from_f32<T>(red[0]);
}

}  // namespace

size_t bias_grad_ws_bytes(const Geom &g)
{
    return size_t((g.B + kIPC - 1) / kIPC) * g.OC * sizeof(float);
}

template <typename T>
hipError_t launch_bias_grad(const Geom &g, const void *dy, const void *ym, void *db, float *part,
                            int relu, hipStream_t s)
{
    const int chunks = (g.B + kIPC - 1) / kIPC;
    const int nt = g.OC >= 256 ? 256 : (g.OC + 63) / 64 * 64;
    const size_t n = size_t(kIPC) * g.OC * g.P;
    if (n <= size_t(kStageMax))   // 256 threads: more loads in flight while staging
        hipLaunchKernelGGL((bias_partials<T, true>), dim3(chunks), dim3(256), n * sizeof(float), s,
                           (const T *)dy, (const T *)ym, part, g, relu);
    else
        hipLaunchKernelGGL((bias_partials<T, false>), dim3(chunks), dim3(nt), 0, s, (const T *)dy,
                           (const T *)ym, part, g, relu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bias_final<T>, dim3(g.OC), dim3(256), 0, s, part, (T *)db, chunks, g.OC);
    return hipGetLastError();
}

template hipError_t launch_bias_grad<float>(const Geom &, const void *, const void *, void *,
                                            float *, int, hipStream_t);
template hipError_t launch_bias_grad<bf16_t>(const Geom &, const void *, const void *, void *,
                                             float *, int, hipStream_t);

}  // namespace gc
