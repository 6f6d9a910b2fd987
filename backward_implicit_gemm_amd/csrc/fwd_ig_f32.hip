// fwd_ig_f32.hip -- forward convolution, fp32 storage, image-group tiling.
//
// Implicit GEMM y[m][n] = sum_k A[m][k] * w[n][k] with m = (b,oh,ow),
// n = oc, k = (ic,kh,kw).  A workgroup owns G whole images (G*OH*OW rows,
// padded to 16-row MFMA blocks) and NW*16*NB output channels; its NW waves
// (eight on the policy-network layers: two per SIMD, so one wave's LDS
// latency hides behind the other's MFMAs) split the channels.  The
// reduction walks input-channel chunks of CC channels: the x planes of the
// G images (CC contiguous NCHW planes per image) and the weight rows (CC*KH*KW
// contiguous weights each) of the next chunk are fetched with 16-byte global
// loads while the MFMAs of the current chunk run, then written to the other
// half of a double-buffered LDS.  The A operand is gathered from the x planes
// through separable offsets held in registers for the whole kernel -- row
// part img*XCS + oh*S*W + ow*S, column part icl*H*W + kh*W + kw -- so no index
// arithmetic remains in the reduction loop.  MFMA: v_mfma_f32_16x16x4_f32,
// fp32 accumulation.  Epilogue: optional ReLU, NCHW store.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

struct FwdIgArgs {
    Geom g;
    const float *x, *w, *bias;
    float *y;
    int relu;
    FwdIgPlan p;
    FastDiv fd_xq;   // XCS/4: float4s per image in the x chunk
    FastDiv fd_wq;   // KCH/4: float4s per weight row in the chunk
};

template <int NW, int MB, int NB, int KS, int XV, int WV>
__global__ void __launch_bounds__(64 * NW) fwd_ig_f32(FwdIgArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const Geom &g = a.g;
    const FwdIgPlan &p = a.p;
    constexpr int NT = 64 * NW;
    constexpr int BN = NW * 16 * NB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const int b0 = blockIdx.x * p.G;
    const int gimg = min(p.G, g.B - b0);
    const int rows = gimg * g.P;
    const int n0 = blockIdx.y * BN;
    const int xbuf = p.G * p.XCS, wbuf = BN * p.KCHP;

    float *xs = lds;                    // [2][G*XCS]
    float *ws = xs + 2 * xbuf;          // [2][BN*KCHP]

    // Weight slots past the chunk (KCH <= k < 4*KS) must read as 0; the
    // staging below never writes them.
    if (4 * KS > p.KCH) {
        const int pad = 4 * KS - p.KCH;
        for (int i = tid; i < 2 * BN * pad; i += NT) {
            const int row = i / pad, k = p.KCH + i % pad;
            ws[row * p.KCHP + k] = 0.f;
        }
    }

    // Column offsets of this lane's k slots, identical for every chunk:
    // k = 4*s + lane/16 -> icl*H*W + kh*W + kw (0 past the chunk's taps,
    // where the weights are zero).
    int koff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int kl = 4 * s + (lane >> 4);
        koff[s] = 0;
        if (kl < p.KCH) {
            uint32_t icl, t, kh, kw;
            fdivmod(kl, g.fd_KK, icl, t);
            fdivmod(t, g.fd_KW, kh, kw);
            koff[s] = int(icl) * g.HW + int(kh) * g.W + int(kw);
        }
    }
    int rowoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = mb * 16 + (lane & 15);
        rowoff[mb] = 0;
        if (r < rows) {
            uint32_t img, pp, oh, ow;
            fdivmod(r, g.fd_P, img, pp);
            fdivmod(pp, g.fd_OW, oh, ow);
            rowoff[mb] = int(img) * p.XCS + int(oh) * g.S * g.W + int(ow) * g.S;
        }
    }

    // Staging: this thread's float4 slots f = tid + NT*j of the x chunk
    // (image, plane offset) and of the weight chunk (row, k offset).  Their
    // positions do not change from chunk to chunk, only the channel base.
    float4 rx[XV], rw[WV];
    const int xq_total = p.G * (p.XCS >> 2), wq_total = BN * (p.KCH >> 2);
    auto fetch = [&](int c) {
        const int c0 = c * p.CC;
        const int valid_x = min(p.CC, g.IC - c0) * g.HW;     // valid floats per image
        const int valid_k = min(p.CC, g.IC - c0) * g.KK;     // valid weights per row
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int f = tid + j * NT;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t img, q;
            fdivmod(f, a.fd_xq, img, q);
            const int e = int(q) * 4;
            if (f < xq_total && int(img) < gimg) {
                const float *src = a.x + (size_t(b0 + int(img)) * g.IC + c0) * g.HW + e;
                if (e + 3 < valid_x) {
                    v = ldg4_any(src);
                } else {
                    if (e + 0 < valid_x) v.x = src[0];
                    if (e + 1 < valid_x) v.y = src[1];
                    if (e + 2 < valid_x) v.z = src[2];
                }
            }
            rx[j] = v;
        }
#pragma unroll
        for (int j = 0; j < WV; ++j) {
            const int f = tid + j * NT;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t n, q;
            fdivmod(f, a.fd_wq, n, q);
            const int kl = int(q) * 4;
            if (f < wq_total && n0 + int(n) < g.OC) {
                const float *src = a.w + size_t(n0 + int(n)) * g.K + size_t(c0) * g.KK + kl;
                if (kl + 3 < valid_k) {
                    v = ldg4_any(src);
                } else {
                    if (kl + 0 < valid_k) v.x = src[0];
                    if (kl + 1 < valid_k) v.y = src[1];
                    if (kl + 2 < valid_k) v.z = src[2];
                }
            }
            rw[j] = v;
        }
    };
    auto stash = [&](int buf) {
        float *xb = xs + buf * xbuf;
        float *wb = ws + buf * wbuf;
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int f = tid + j * NT;
            if (f < xq_total) {
                uint32_t img, q;
                fdivmod(f, a.fd_xq, img, q);
                *reinterpret_cast<float4 *>(xb + int(img) * p.XCS + int(q) * 4) = rx[j];
            }
        }
#pragma unroll
        for (int j = 0; j < WV; ++j) {
            const int f = tid + j * NT;
            if (f < wq_total) {
                uint32_t n, q;
                fdivmod(f, a.fd_wq, n, q);
                float2 *d = reinterpret_cast<float2 *>(wb + int(n) * p.KCHP + int(q) * 4);
                d[0] = make_float2(rw[j].x, rw[j].y);
                d[1] = make_float2(rw[j].z, rw[j].w);
            }
        }
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    fetch(0);
    stash(0);
    __syncthreads();
    const int ncol0 = wave * NB * 16 + (lane & 15);
    for (int c = 0; c < p.nchunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < p.nchunks) fetch(c + 1);
        const float *xb = xs + buf * xbuf;
        const float *wb = ws + buf * wbuf + ncol0 * p.KCHP + (lane >> 4);
        const float *xr[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xr[mb] = xb + rowoff[mb];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float av[MB], bv[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) av[mb] = xr[mb][koff[s]];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) bv[nb] = wb[nb * 16 * p.KCHP + s * 4];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
        }
        if (c + 1 < p.nchunks) stash(buf ^ 1);
        __syncthreads();
    }

    // epilogue: row r = mb*16 + 4*(lane/16) + v, column n0 + wave*16*NB + nb*16 + lane%16
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = mb * 16 + (lane >> 4) * 4 + v;
            if (r >= rows) continue;
            uint32_t img, pp;
            fdivmod(r, g.fd_P, img, pp);
            float *yrow = a.y + size_t(b0 + int(img)) * g.OC * g.P + int(pp);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int n = n0 + ncol0 + nb * 16;
                if (n >= g.OC) continue;
                float val = acc[mb][nb][v];
                if (a.bias) val += a.bias[n];
                if (a.relu && !(val > 0.f)) val = 0.f;
                yrow[size_t(n) * g.P] = val;
            }
        }
}

// Instantiated tilings: (NW, MB, NB, KS, XV, WV).
struct FwdVariant {
    int NW, MB, NB, KS, XV, WV;
    void (*fn)(FwdIgArgs);
};

#define FWD_V(NW, MB, NB, KS, XV, WV) {NW, MB, NB, KS, XV, WV, fwd_ig_f32<NW, MB, NB, KS, XV, WV>}
const FwdVariant kFwdVariants[] = {
    FWD_V(8, 3, 1, 25, 2, 7),    // layer 1: 4 images of 3x4 outputs, 4 channels x 25 taps
    FWD_V(4, 1, 1, 36, 2, 9),    // layer 2: 8 images of 1x2 outputs, 16 channels x 9 taps
    FWD_V(8, 4, 1, 36, 3, 9),    // layer 2 at large batch: 32 images
    FWD_V(8, 1, 1, 25, 2, 7), FWD_V(8, 2, 1, 25, 2, 7), FWD_V(8, 4, 1, 25, 2, 7),
    FWD_V(4, 1, 1, 25, 2, 7), FWD_V(4, 2, 1, 25, 2, 7), FWD_V(4, 3, 1, 25, 2, 7),
    FWD_V(4, 4, 1, 25, 2, 7),
    FWD_V(4, 1, 1, 16, 2, 5), FWD_V(4, 2, 1, 16, 2, 5), FWD_V(4, 3, 1, 16, 2, 5),
    FWD_V(4, 4, 1, 16, 2, 5),
    FWD_V(8, 1, 1, 16, 2, 5), FWD_V(8, 2, 1, 16, 2, 5), FWD_V(8, 3, 1, 16, 2, 5),
    FWD_V(8, 4, 1, 16, 2, 5),
    FWD_V(4, 2, 1, 36, 2, 9), FWD_V(4, 3, 1, 36, 2, 9), FWD_V(4, 4, 1, 36, 2, 9),
    FWD_V(8, 1, 1, 36, 2, 5), FWD_V(8, 2, 1, 36, 2, 5), FWD_V(8, 3, 1, 36, 2, 5),
};
#undef FWD_V

int round_up(int v, int m) { return (v + m - 1) / m * m; }

const FwdVariant *pick_fwd(int NW, int MB, int kch, int xv, int wv)
{
    const FwdVariant *best = nullptr;
    for (const auto &v : kFwdVariants)
        if (v.NW == NW && v.MB == MB && v.NB == 1 && 4 * v.KS >= kch && xv <= v.XV &&
            wv <= v.WV && (!best || v.KS < best->KS))
            best = &v;
    return best;
}

}  // namespace

// Chooses G, the tile width and the channel chunk; false when the shape does
// not fit this kernel (the shape-generic kernel then runs).
bool plan_fwd_ig_f32(const Geom &g, FwdIgPlan &p)
{
    if (g.P > 64) return false;
    // Eight waves (128 channels) unless the grid would then be too small to
    // fill the chip (layer-2-like problems with 2 rows per image).
    const size_t budget = 150 * 1024;
    bool found = false;
    double best = -1.0;
    for (int NW : {8, 4}) {
        const int BN = NW * 16;
        const int ntile_n = (g.OC + BN - 1) / BN;
        int G = 64 / g.P;
        while (G > 1 && ((g.B + G - 1) / G) * ntile_n < 256) --G;
        if (g.P == 12 && G > 4) G = 4;
        if (NW == 8 && ((g.B + G - 1) / G) * ntile_n < 256 && g.OC <= 64) continue;
        if (NW == 8 && g.P <= 4 && g.B * g.P < 256 * 64) continue;
        const int MB = (G * g.P + 15) / 16;
        for (int CC = std::min(g.IC, 16); CC >= 1; --CC) {
            if ((CC * g.KK) % 4) continue;     // float4 weight staging
            FwdIgPlan q;
            q.NW = NW; q.G = G; q.MB = MB; q.NB = 1; q.CC = CC;
            q.KCH = CC * g.KK;
            q.XCS = round_up(CC * g.HW, 4);
            q.nchunks = (g.IC + CC - 1) / CC;
            q.XV = (G * q.XCS / 4 + 64 * NW - 1) / (64 * NW);
            q.WV = (BN * (q.KCH / 4) + 64 * NW - 1) / (64 * NW);
            const FwdVariant *v = pick_fwd(NW, MB, q.KCH, q.XV, q.WV);
            if (!v) continue;
            q.KS = v->KS;
            // weight rows hold 4*KS slots (zero past KCH); a stride of 2 mod 4
            // puts the 16 rows an MFMA B operand reads on distinct LDS banks
            q.KCHP = round_up(4 * q.KS, 4) + 2;
            q.lds = sizeof(float) * (2 * size_t(G) * q.XCS + 2 * size_t(BN) * q.KCHP);
            if (q.lds > budget) continue;
            const double eff = double(q.KCH) / (4 * q.KS);
            if (eff > best + 1e-9) {
                best = eff;
                p = q;
                found = true;
            }
        }
        if (found) break;
    }
    return found;
}

hipError_t launch_fwd_ig_f32(const Geom &g, const FwdIgPlan &p, const void *x, const void *w,
                             const void *bias, void *y, int relu, hipStream_t s)
{
    const FwdVariant *v = pick_fwd(p.NW, p.MB, p.KCH, p.XV, p.WV);
    if (!v || v->KS != p.KS || 4 * p.KS + 2 > p.KCHP) return hipErrorInvalidValue;
    FwdIgArgs a{g, (const float *)x, (const float *)w, (const float *)bias, (float *)y, relu, p,
                make_fastdiv(p.XCS / 4), make_fastdiv(p.KCH / 4)};
    dim3 grid((g.B + p.G - 1) / p.G, (g.OC + 16 * p.NW - 1) / (16 * p.NW));
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
