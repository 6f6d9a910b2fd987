// igemm_generic.hip -- shape-generic implicit-GEMM kernels for the three
// convolution passes (forward, d_input, wgrad) on gfx950 MFMA.
//
// Each pass is a GEMM C[M][N] = sum_k A[m][k] * B[k][n] whose operands are
// never materialised in HBM: a 64x64 workgroup tile walks the reduction in
// chunks of 32, gathers the A and B chunk elements straight from the NCHW /
// OIHW tensors through the magic-number index mapper into LDS (k-contiguous
// rows), and feeds them to MFMA (v_mfma_f32_16x16x4_f32 for fp32 storage,
// v_mfma_f32_16x16x32_bf16 for bf16 storage; fp32 accumulation in both).
// The next chunk's global loads are issued before the current chunk's MFMAs.
//
//   forward : M = B*OH*OW (b,oh,ow)   N = OC   K = IC*KH*KW (ic,kh,kw)
//   d_input : M = B*H*W   (b,ih,iw)   N = IC   K = OC*KH*KW (oc,kh,kw), taps
//             that do not land on an output position read as zero, so every
//             dx element is produced by exactly one workgroup (no atomics)
//   wgrad   : M = OC                  N = IC*KH*KW        K = B*OH*OW, split
//             across grid.z into fp32 partials, then a fixed-order sum
//
// These kernels serve every shape the API accepts; the layer shapes of the
// policy network get the specialised kernels in the other sources.
#include "gc_common.h"
#include "gc_kernels.h"

namespace gc {
namespace {

constexpr int TM = 64;     // tile rows
constexpr int TN = 64;     // tile columns
constexpr int KC = 32;     // reduction chunk
constexpr int NT = 256;    // threads per workgroup (4 waves, 2x2 of 32x32)
constexpr int RPT = TM * KC / NT;   // rows each thread stages per chunk (8)

template <typename T> struct Lds;
template <> struct Lds<float> { static constexpr int PAD = 1; };
template <> struct Lds<bf16_t> { static constexpr int PAD = 8; };

// ----------------------------------------------------------------- ops ----
// Each op splits an operand element into a row part and a column part so
// that per-row and per-column index math is done once per tile / per chunk.

template <typename T>
struct FwdOp {
    Geom g; const T *x, *w, *bias; T *y; int relu;
    __device__ int M() const { return g.B * g.P; }
    __device__ int N() const { return g.OC; }
    __device__ int K() const { return g.K; }
    // A[m][k] = x[b, ic, oh*S+kh, ow*S+kw]
    __device__ int a_row(int m) const {
        if (m >= M()) return -1;
        uint32_t b, p, oh, ow;
        fdivmod(m, g.fd_P, b, p);
        fdivmod(p, g.fd_OW, oh, ow);
        return int(b) * g.IC * g.HW + int(oh) * g.S * g.W + int(ow) * g.S;
    }
    __device__ int a_col(int k) const {
        if (k >= g.K) return -1;
        uint32_t ic, t, kh, kw;
        fdivmod(k, g.fd_KK, ic, t);
        fdivmod(t, g.fd_KW, kh, kw);
        return int(ic) * g.HW + int(kh) * g.W + int(kw);
    }
    __device__ T a_load(int r, int c) const { return (r < 0 || c < 0) ? T(0) : x[r + c]; }
    // B stored as [n][k]: w[n, k]
    __device__ int b_row(int n) const { return n < g.OC ? n * g.K : -1; }
    __device__ int b_col(int k) const { return k < g.K ? k : -1; }
    __device__ T b_load(int r, int c) const { return (r < 0 || c < 0) ? T(0) : w[r + c]; }
    __device__ void store(int m, int n, float v) const {
        uint32_t b, p;
        fdivmod(m, g.fd_P, b, p);
        if (bias) v += to_f32(bias[n]);
        if (relu && !(v > 0.f)) v = 0.f;
        y[(int(b) * g.OC + n) * g.P + int(p)] = from_f32<T>(v);
    }
};

template <typename T>
struct DgradOp {
    Geom g; const T *dy, *w, *ym; T *dx; int relu;
    __device__ int M() const { return g.B * g.HW; }
    __device__ int N() const { return g.IC; }
    __device__ int K() const { return g.OC * g.KK; }
    // A[pix][(oc,kh,kw)] = dz[b, oc, (ih-kh)/S, (iw-kw)/S] when that tap lands
    // on an output position, else 0.  Row part packs (b, ih, iw).
    struct Row { int b, ih, iw; };
    __device__ Row a_row(int pix) const {
        if (pix >= M()) return Row{-1, 0, 0};
        uint32_t b, q, ih, iw;
        fdivmod(pix, g.fd_HW, b, q);
        fdivmod(q, g.fd_W, ih, iw);
        return Row{int(b), int(ih), int(iw)};
    }
    struct Col { int oc, kh, kw; };
    __device__ Col a_col(int k) const {
        if (k >= K()) return Col{-1, 0, 0};
        uint32_t oc, t, kh, kw;
        fdivmod(k, g.fd_KK, oc, t);
        fdivmod(t, g.fd_KW, kh, kw);
        return Col{int(oc), int(kh), int(kw)};
    }
    __device__ T a_load(const Row &r, const Col &c) const {
        if (r.b < 0 || c.oc < 0) return T(0);
        const int th = r.ih - c.kh, tw = r.iw - c.kw;
        if (th < 0 || tw < 0) return T(0);
        uint32_t oh, rh, ow, rw;
        fdivmod(th, g.fd_S, oh, rh);
        fdivmod(tw, g.fd_S, ow, rw);
        if (rh | rw) return T(0);
        if (int(oh) >= g.OH || int(ow) >= g.OW) return T(0);
        const int i = (r.b * g.OC + c.oc) * g.P + int(oh) * g.OW + int(ow);
        if (relu && !(to_f32(ym[i]) > 0.f)) return T(0);
        return dy[i];
    }
    // B stored as [ic][(oc,kh,kw)]: w[oc, ic, kh, kw]
    __device__ int b_row(int ic) const { return ic < g.IC ? ic * g.KK : -1; }
    __device__ int b_col(int k) const {
        if (k >= K()) return -1;
        uint32_t oc, t;
        fdivmod(k, g.fd_KK, oc, t);
        return int(oc) * g.K + int(t);
    }
    __device__ T b_load(int r, int c) const { return (r < 0 || c < 0) ? T(0) : w[r + c]; }
    __device__ void store(int pix, int ic, float v) const {
        uint32_t b, q;
        fdivmod(pix, g.fd_HW, b, q);
        dx[(int(b) * g.IC + ic) * g.HW + int(q)] = from_f32<T>(v);
    }
};

template <typename T>
struct WgradOp {
    Geom g; const T *x, *dy, *ym; float *part; int relu;
    __device__ int M() const { return g.OC; }
    __device__ int N() const { return g.K; }
    __device__ int K() const { return g.B * g.P; }
    // A[oc][r] = dz[b, oc, p] with r = (b, p)
    __device__ int a_row(int oc) const { return oc < g.OC ? oc * g.P : -1; }
    __device__ int a_col(int r) const {
        if (r >= K()) return -1;
        uint32_t b, p;
        fdivmod(r, g.fd_P, b, p);
        return int(b) * g.OC * g.P + int(p);
    }
    __device__ T a_load(int rr, int cc) const {
        if (rr < 0 || cc < 0) return T(0);
        const int i = rr + cc;
        if (relu && !(to_f32(ym[i]) > 0.f)) return T(0);
        return dy[i];
    }
    // B stored as [(ic,kh,kw)][r]: x[b, ic, oh*S+kh, ow*S+kw]
    __device__ int b_row(int k) const {
        if (k >= g.K) return -1;
        uint32_t ic, t, kh, kw;
        fdivmod(k, g.fd_KK, ic, t);
        fdivmod(t, g.fd_KW, kh, kw);
        return int(ic) * g.HW + int(kh) * g.W + int(kw);
    }
    __device__ int b_col(int r) const {
        if (r >= K()) return -1;
        uint32_t b, p, oh, ow;
        fdivmod(r, g.fd_P, b, p);
        fdivmod(p, g.fd_OW, oh, ow);
        return int(b) * g.IC * g.HW + int(oh) * g.S * g.W + int(ow) * g.S;
    }
    __device__ T b_load(int rr, int cc) const { return (rr < 0 || cc < 0) ? T(0) : x[rr + cc]; }
    __device__ void store_split(int split, int oc, int k, float v) const {
        part[(size_t(split) * g.OC + oc) * g.K + k] = v;
    }
};

// -------------------------------------------------------------- MFMA ----

__device__ __forceinline__ void mma_chunk(const float *As, const float *Bs, f32x4 (&acc)[2][2],
                                          int wm, int wn, int lane)
{
    constexpr int LD = KC + Lds<float>::PAD;
#pragma unroll
    for (int ks = 0; ks < KC / 4; ++ks) {
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a[i] = As[(wm * 32 + i * 16 + (lane & 15)) * LD + ks * 4 + (lane >> 4)];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j] = Bs[(wn * 32 + j * 16 + (lane & 15)) * LD + ks * 4 + (lane >> 4)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

__device__ __forceinline__ void mma_chunk(const bf16_t *As, const bf16_t *Bs, f32x4 (&acc)[2][2],
                                          int wm, int wn, int lane)
{
    constexpr int LD = KC + Lds<bf16_t>::PAD;
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * 32 + i * 16 + (lane & 15)) * LD + (lane >> 4) * 8]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * 32 + j * 16 + (lane & 15)) * LD + (lane >> 4) * 8]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// ------------------------------------------------------------ kernel ----
// grid = (ceil(M/64), ceil(N/64), splits); blockIdx.z covers reduction range
// [z*kspan, min((z+1)*kspan, K)).  `Final` selects the epilogue.

template <typename T, class Op>
__device__ __forceinline__ void tile_gemm(const Op &op, int kspan, f32x4 (&acc)[2][2],
                                          int &m0, int &n0)
{
    constexpr int LD = KC + Lds<T>::PAD;
    __shared__ __attribute__((aligned(16))) T As[TM * LD];
    __shared__ __attribute__((aligned(16))) T Bs[TN * LD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    m0 = blockIdx.x * TM;
    n0 = blockIdx.y * TN;
    const int kbeg = blockIdx.z * kspan;
    const int kend = min(kbeg + kspan, op.K());

    const int kl = tid % KC, r0 = tid / KC;

    // Row parts of this thread's staged rows, fixed for the whole tile.
    decltype(op.a_row(0)) ra[RPT];
    decltype(op.b_row(0)) rb[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        ra[j] = op.a_row(m0 + r0 + j * (NT / KC));
        rb[j] = op.b_row(n0 + r0 + j * (NT / KC));
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    T va[RPT], vb[RPT];
    auto fetch = [&](int k0) {
        const int k = k0 + kl;
        const bool in = k < kend;
        const auto ca = op.a_col(in ? k : op.K());
        const auto cb = op.b_col(in ? k : op.K());
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            va[j] = op.a_load(ra[j], ca);
            vb[j] = op.b_load(rb[j], cb);
        }
    };

    if (kbeg < kend) fetch(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += KC) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            As[(r0 + j * (NT / KC)) * LD + kl] = va[j];
            Bs[(r0 + j * (NT / KC)) * LD + kl] = vb[j];
        }
        __syncthreads();
        if (k0 + KC < kend) fetch(k0 + KC);
        mma_chunk(As, Bs, acc, wm, wn, lane);
    }
}

template <typename T>
__global__ void __launch_bounds__(NT) fwd_generic(FwdOp<T> op)
{
    f32x4 acc[2][2];
    int m0, n0;
    tile_gemm<T>(op, op.K(), acc, m0, n0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + v;
                const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                if (m < op.M() && n < op.N()) op.store(m, n, acc[i][j][v]);
            }
}

template <typename T>
__global__ void __launch_bounds__(NT) dgrad_generic(DgradOp<T> op)
{
    f32x4 acc[2][2];
    int m0, n0;
    tile_gemm<T>(op, op.K(), acc, m0, n0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + v;
                const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                if (m < op.M() && n < op.N()) op.store(m, n, acc[i][j][v]);
            }
}

template <typename T>
__global__ void __launch_bounds__(NT) wgrad_generic(WgradOp<T> op, int kspan)
{
    f32x4 acc[2][2];
    int m0, n0;
    tile_gemm<T>(op, kspan, acc, m0, n0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + v;
                const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                if (m < op.M() && n < op.N()) op.store_split(blockIdx.z, m, n, acc[i][j][v]);
            }
}

}  // namespace

// ------------------------------------------------------------ launch ----

template <typename T>
hipError_t launch_fwd_generic(const Geom &g, const void *x, const void *w, const void *bias,
                              void *y, int relu, hipStream_t s)
{
    FwdOp<T> op{g, (const T *)x, (const T *)w, (const T *)bias, (T *)y, relu};
    dim3 grid((g.B * g.P + TM - 1) / TM, (g.OC + TN - 1) / TN, 1);
    hipLaunchKernelGGL(fwd_generic<T>, grid, dim3(NT), 0, s, op);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dgrad_generic(const Geom &g, const void *dy, const void *w, const void *ym,
                                void *dx, int relu, hipStream_t s)
{
    DgradOp<T> op{g, (const T *)dy, (const T *)w, (const T *)ym, (T *)dx, relu};
    dim3 grid((g.B * g.HW + TM - 1) / TM, (g.IC + TN - 1) / TN, 1);
    hipLaunchKernelGGL(dgrad_generic<T>, grid, dim3(NT), 0, s, op);
    return hipGetLastError();
}

int wgrad_generic_splits(const Geom &g)
{
    const int tiles = ((g.OC + TM - 1) / TM) * ((g.K + TN - 1) / TN);
    const int R = g.B * g.P;
    const int max_by_len = (R + KC - 1) / KC;          // at least one chunk per split
    int want = (1024 + tiles - 1) / tiles;             // aim for ~4 workgroups per CU
    if (want > 64) want = 64;
    if (want > max_by_len) want = max_by_len;
    return want < 1 ? 1 : want;
}

int wgrad_generic_kspan(const Geom &g, int splits)
{
    const int R = g.B * g.P;
    int span = (R + splits - 1) / splits;
    return (span + KC - 1) / KC * KC;
}

template <typename T>
hipError_t launch_wgrad_generic(const Geom &g, const void *x, const void *dy, const void *ym,
                                float *part, int splits, int relu, hipStream_t s)
{
    WgradOp<T> op{g, (const T *)x, (const T *)dy, (const T *)ym, part, relu};
    const int kspan = wgrad_generic_kspan(g, splits);
    dim3 grid((g.OC + TM - 1) / TM, (g.K + TN - 1) / TN, splits);
    hipLaunchKernelGGL(wgrad_generic<T>, grid, dim3(NT), 0, s, op, kspan);
    return hipGetLastError();
}

template hipError_t launch_fwd_generic<float>(const Geom &, const void *, const void *, const void *,
                                              void *, int, hipStream_t);
template hipError_t launch_fwd_generic<bf16_t>(const Geom &, const void *, const void *, const void *,
                                              void *, int, hipStream_t);
template hipError_t launch_dgrad_generic<float>(const Geom &, const void *, const void *, const void *, void *, int, hipStream_t);
template hipError_t launch_dgrad_generic<bf16_t>(const Geom &, const void *, const void *, const void *, void *, int, hipStream_t);
template hipError_t launch_wgrad_generic<float>(const Geom &, const void *, const void *, const void *, float *, int, int, hipStream_t);
template hipError_t launch_wgrad_generic<bf16_t>(const Geom &, const void *, const void *, const void *, float *, int, int, hipStream_t);

}  // namespace gc
