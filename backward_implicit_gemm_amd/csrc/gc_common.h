// gc_common.h -- shared pieces of the gfx950 kernels: the magic-number index
// mapper, the problem geometry handed to every kernel, and bf16 helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gc {

// ---------------------------------------------------------------------------
// Division by an invariant integer without a hardware divide.
//
// Granlund & Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994): for a divisor d >= 1 let s = ceil(log2 d) and
// m = floor(2^32 * (2^s - d) / d) + 1 (which fits in 32 bits because
// 2^s - d < d).  Then for 0 <= n < 2^31
//     q = (umulhi(n, m) + n) >> s,   r = n - q * d.
// umulhi(n, m) < n, so the 32-bit sum cannot wrap for n < 2^31.  The pull
// request this library follows credits its speedup to a fast divmod of this
// kind plus caching of repeated index math; here the divisors of a call are
// prepared once on the host and every (b,oh,ow) / (ic,kh,kw) split in the
// kernels is two multiplies and a shift.
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t d;      // divisor
    uint32_t mul;    // m above
    uint32_t shift;  // s above
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
    return FastDiv{d, uint32_t(m), s};
}

__host__ __device__ __forceinline__ uint32_t umulhi32(uint32_t a, uint32_t b)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __umulhi(a, b);
#else
    return uint32_t((uint64_t(a) * b) >> 32);
#endif
}

__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f)
{
    return (umulhi32(n, f.mul) + n) >> f.shift;
}

// q = n / d, r = n % d
__host__ __device__ __forceinline__ void fdivmod(uint32_t n, const FastDiv &f,
                                                 uint32_t &q, uint32_t &r)
{
    q = fdiv(n, f);
    r = n - q * f.d;
}

// ---------------------------------------------------------------------------
// Geometry of one convolution call, passed by value to the kernels.
// ---------------------------------------------------------------------------
struct Geom {
    int B, IC, H, W, OC, KH, KW, S, OH, OW;
    int P;    // OH*OW, output positions per image
    int KK;   // KH*KW, taps per channel
    int HW;   // H*W, pixels per channel plane
    int K;    // IC*KK, reduction length of the forward GEMM
    FastDiv fd_P, fd_OW, fd_KK, fd_KW, fd_HW, fd_W, fd_S, fd_OC;
    // the device the call runs on: compute units, and the XCDs (each with its
    // own L2) that workgroup ids are dealt to round-robin.  Plans size their
    // grids from these; kernels use nxcd only to place related workgroups on
    // one XCD, never for coverage.
    int ncu, nxcd;
};

inline Geom make_geom(int B, int IC, int H, int W, int OC, int KH, int KW, int S)
{
    Geom g;
    g.B = B; g.IC = IC; g.H = H; g.W = W; g.OC = OC; g.KH = KH; g.KW = KW; g.S = S;
    g.OH = (H - KH) / S + 1;
    g.OW = (W - KW) / S + 1;
    g.P = g.OH * g.OW;
    g.KK = KH * KW;
    g.HW = H * W;
    g.K = IC * g.KK;
    g.fd_P = make_fastdiv(g.P);
    g.fd_OW = make_fastdiv(g.OW);
    g.fd_KK = make_fastdiv(g.KK);
    g.fd_KW = make_fastdiv(KW);
    g.fd_HW = make_fastdiv(g.HW);
    g.fd_W = make_fastdiv(W);
    g.fd_S = make_fastdiv(S);
    g.fd_OC = make_fastdiv(OC);
    g.ncu = 256;     // MI355X; the C ABI layer sets the current device's values
    g.nxcd = 8;
    return g;
}

// ---------------------------------------------------------------------------
// Storage types.  bf16 travels as its 16-bit pattern; widening to fp32 is a
// shift, narrowing rounds to nearest even through the compiler's __bf16
// conversion (a hardware convert on gfx950).
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v)
{
    __bf16 h = (__bf16)v;
    return __builtin_bit_cast(bf16_t, h);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

}  // namespace gc
