// fwd_rf_f32.hip -- forward convolution, fp32 storage, fp32 MFMA
// (v_mfma_f32_16x16x4_f32), operands laid out so one 16-byte read feeds four
// MFMA steps.
//
// Implicit GEMM y[m][n] = sum_k A[m][k] * w[n][k], m = (b,oh,ow), n = oc.  The
// reduction runs in blocks of 16 k = 4 channels x 4 taps: in block (channel
// group cg, tap step s), MFMA step j (0..3) gives lane group q = lane/16 the
// element (channel 4*cg + j, tap 4*s + q).  So a lane's four steps read four
// consecutive channels at one tap, and both operands come as float4:
//   * x: a workgroup owns G whole images; channel groups are staged in LDS
//     channels-innermost, [group][image][pixel][4 channels], through 4x4
//     register transposes, so the A operand of output row (b,oh,ow) at tap
//     (kh,kw) for four steps is the 16 bytes at pixel (oh*S+kh, ow*S+kw);
//   * w: a small pre-pass packs the weights into that order --
//     [16-channel block][channel group][tap step][lane] x 4 channels -- and
//     each wave streams its 16 output channels' fragments from L2 through a
//     ring of 16 registers, unrolled at compile time.
// Channel groups are staged in NPH phases through two LDS buffers: the loads
// of phase ph+1 are in flight while phase ph's MFMAs run.  Channels are padded
// to a multiple of 4 and taps to a multiple of 4 with zero weights.
// Epilogue: optional bias and ReLU, NCHW store.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {

void pick_lds_pitch(const Geom &g, int G, int MB, int TS, int &WP_out, int &IS_out);

namespace {

// Packed weights, 16-byte units ((nb*NCG + cg)*TS + s)*64 + lane holding
// w[16*nb + lane%16][4*cg + j][4*s + lane/16] for j = 0..3 (zero past OC, IC
// or KH*KW).
__global__ void __launch_bounds__(256) pack_w_fwd_f32(const float *__restrict__ w,
                                                      float4 *__restrict__ wf, Geom g, int NCG,
                                                      int TS, int total)
{
    for (int u = blockIdx.x * 256 + threadIdx.x; u < total; u += gridDim.x * 256) {
        const int lane = u & 63;
        int rest = u >> 6;
        const int s = rest % TS;
        rest /= TS;
        const int cg = rest % NCG;
        const int nb = rest / NCG;
        const int n = nb * 16 + (lane & 15);
        const int t = 4 * s + (lane >> 4);
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ic = 4 * cg + j;
            v[j] = (n < g.OC && ic < g.IC && t < g.KK) ? w[(size_t(n) * g.IC + ic) * g.KK + t] : 0.f;
        }
        wf[u] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

struct FwdRfArgs {
    Geom g;
    const float *x;
    const float4 *wf;
    const float *bias;
    float *y;
    int relu;
    int G;        // images per workgroup
    int WP;       // LDS pixel slots per image row (>= W)
    int IS;       // LDS pixel slots per image (>= H*WP)
    int nblk;     // 4-pixel blocks per image plane
};

__device__ __forceinline__ float comp(const float4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int NW, int MB, int TS, int NCG, int NPH, int D>
__global__ void __launch_bounds__(64 * NW) fwd_rf_f32(FwdRfArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float4 lds4f[];
    const Geom &g = a.g;
    constexpr int BN = 16 * NW;
    constexpr int NFRAG = NCG * TS;
    constexpr int CPP = (NCG + NPH - 1) / NPH;      // channel groups per staging phase
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b0 = blockIdx.x * a.G;
    const int gimg = min(a.G, g.B - b0);
    const int rows = gimg * g.P;
    const int n0 = blockIdx.y * BN;
    const int nb = blockIdx.y * NW + wave;          // 16-channel block of this wave
    const int gstride = a.G * a.IS;                 // float4 slots per channel group in LDS
    const int bufsz = CPP * gstride;                // one phase buffer

    // weight fragments through a ring of D registers (see the header)
    const float4 *wf_wave = a.wf + size_t(nb) * NFRAG * 64 + lane;
    float4 ring[D];
#pragma unroll
    for (int j = 0; j < D; ++j)
        ring[j] = j < NFRAG ? wf_wave[size_t(j) * 64] : make_float4(0.f, 0.f, 0.f, 0.f);

    // x staging, one unit per thread per phase: unit u = (cgl, img, 4-pixel
    // block) of the phase's channel groups: 4 loads of 4 pixels (one per
    // channel), a 4x4 transpose, 4 stores of 4 channels.  Images past the
    // batch and channels past IC get zeros.
    const int units_per_cg = a.G * a.nblk;
    float4 in[4];
    int u_cgl = 0, u_img = 0, u_pix = 0, u_npix = 0, u_cg = 0;
    bool u_on = false;
    auto fetch_x = [&](int ph) {
        const int cg0 = ph * CPP;
        const int ncg = min(CPP, NCG - cg0);
        const int u = tid;
        u_on = u < ncg * units_per_cg;
        const int blk = u % a.nblk;
        const int rest = u / a.nblk;
        u_img = rest % a.G;
        u_cgl = rest / a.G;
        u_cg = cg0 + u_cgl;
        u_pix = blk * 4;
        u_npix = min(4, g.HW - u_pix);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ic = u_cg * 4 + c;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u_on && u_img < gimg && ic < g.IC) {
                const float *src = a.x + (size_t(b0 + u_img) * g.IC + ic) * g.HW + u_pix;
                if (u_npix == 4) {
                    __builtin_memcpy(&v, src, 16);
                } else {
                    float e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) e[i] = i < u_npix ? src[i] : 0.f;
                    v = make_float4(e[0], e[1], e[2], e[3]);
                }
            }
            in[c] = v;
        }
    };
    auto stash_x = [&](int buf) {
        if (!u_on) return;
        float4 *dst = lds4f + buf * bufsz + u_cgl * gstride + u_img * a.IS;
        int ih = u_pix / g.W, iw = u_pix - ih * g.W;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            const float4 o = make_float4(comp(in[0], pp), comp(in[1], pp), comp(in[2], pp), comp(in[3], pp));
            if (pp < u_npix) dst[ih * a.WP + iw] = o;
            if (++iw == g.W) { iw = 0; ++ih; }
        }
    };

    // LDS pixel offsets (16-byte slots) of this lane's A rows and taps
    int rowoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = mb * 16 + (lane & 15);
        rowoff[mb] = 0;
        if (r < rows) {
            uint32_t img, pp, oh, ow;
            fdivmod(r, g.fd_P, img, pp);
            fdivmod(pp, g.fd_OW, oh, ow);
            rowoff[mb] = int(img) * a.IS + int(oh) * g.S * a.WP + int(ow) * g.S;
        }
    }
    int toff[TS];
#pragma unroll
    for (int s = 0; s < TS; ++s) {
        const int t = 4 * s + (lane >> 4);
        toff[s] = 0;
        if (t < g.KK) {
            uint32_t kh, kw;
            fdivmod(t, g.fd_KW, kh, kw);
            toff[s] = int(kh) * a.WP + int(kw);
        }
    }

    f32x4 acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    fetch_x(0);
    stash_x(0);
    __syncthreads();
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        if (ph + 1 < NPH) fetch_x(ph + 1);       // next phase's loads fly during this one
        const float4 *xbuf = lds4f + (ph & 1) * bufsz;
#pragma unroll
        for (int cg = ph * CPP; cg < (ph + 1) * CPP && cg < NCG; ++cg) {
            // all A fragments of the channel group first, then its MFMAs
            const float4 *xb = xbuf + (cg - ph * CPP) * gstride;
            float4 af[TS][MB];
#pragma unroll
            for (int st = 0; st < TS; ++st)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) af[st][mb] = xb[rowoff[mb] + toff[st]];
#pragma unroll
            for (int st = 0; st < TS; ++st) {
                const int f = cg * TS + st;
                const float4 bv = ring[f % D];
                if (f + D < NFRAG) ring[f % D] = wf_wave[size_t(f + D) * 64];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(af[st][mb], j), comp(bv, j),
                                                                       acc[mb], 0, 0, 0);
            }
        }
        if (ph + 1 < NPH) {
            stash_x((ph + 1) & 1);
            __syncthreads();
        }
    }

    // epilogue: row r = mb*16 + 4*(lane/16) + v, column n0 + wave*16 + lane%16
    const int n = n0 + wave * 16 + (lane & 15);
    if (n < g.OC) {
        const float bn = a.bias ? a.bias[n] : 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = mb * 16 + (lane >> 4) * 4 + v;
                if (r >= rows) continue;
                uint32_t img, pp;
                fdivmod(r, g.fd_P, img, pp);
                float val = acc[mb][v] + bn;
                if (a.relu && !(val > 0.f)) val = 0.f;
                a.y[(size_t(b0 + int(img)) * g.OC + n) * g.P + int(pp)] = val;
            }
    }
}

struct FwdRfVariant {
    int NW, MB, TS, NCG, NPH;
    void (*fn)(FwdRfArgs);
};

constexpr int kRingF = 16;   // weight fragments in flight per lane
#define FR_V(NW, MB, TS, NCG, NPH) {NW, MB, TS, NCG, NPH, fwd_rf_f32<NW, MB, TS, NCG, NPH, kRingF>}
const FwdRfVariant kFwdRfVariants[] = {
    FR_V(8, 3, 7, 15, 5),    // layer 1: 4 images x 12 rows, 25 taps (7 steps), 59 -> 60 channels
    FR_V(8, 1, 7, 15, 5),    // layer 1, fewer than 4 images per workgroup
    FR_V(4, 4, 3, 32, 16),   // layer 2: 32 images x 2 rows, 9 taps (3 steps), 128 channels
    FR_V(4, 1, 3, 32, 16),   // layer 2, 8 or fewer images
    FR_V(4, 2, 3, 32, 16), FR_V(4, 3, 3, 32, 16),
};
#undef FR_V

// A variant whose staging phases give every unit a thread: NPH phases of
// ceil(NCG/NPH) channel groups x G images x nblk pixel blocks each.
const FwdRfVariant *pick_fwd_rf(int NW, int MB, int TS, int NCG, int units_per_cg)
{
    for (const auto &v : kFwdRfVariants)
        if (v.NW == NW && v.MB == MB && v.TS == TS && v.NCG == NCG &&
            (NCG + v.NPH - 1) / v.NPH * units_per_cg <= 64 * NW)
            return &v;
    return nullptr;
}

}  // namespace

bool plan_fwd_rf_f32(const Geom &g, FwdBfPlan &p)
{
    if (g.P > 64 || g.KK > 36) return false;
    const int TS = (g.KK + 3) / 4;
    const int order[2] = {g.P <= 4 ? 4 : 8, g.P <= 4 ? 8 : 4};
    for (int NW : order) {
        const int BN = 16 * NW;
        const int ntile_n = (g.OC + BN - 1) / BN;
        int G = std::max(1, 64 / g.P);
        while (G > 1 && ((g.B + G - 1) / G) * ntile_n < 256) --G;
        if (g.P == 12 && G > 4) G = 4;
        if (G > g.B) G = g.B;
        const int MB = (G * g.P + 15) / 16;
        FwdBfPlan q;
        q.NW = NW; q.G = G; q.MB = MB; q.TS = TS;
        q.nblk = (g.HW + 3) / 4;
        q.NCG = (g.IC + 3) / 4;
        pick_lds_pitch(g, G, MB, TS, q.WP, q.IS);
        const FwdRfVariant *v = pick_fwd_rf(NW, MB, TS, q.NCG, G * q.nblk);
        if (!v) continue;
        const int CPP = (q.NCG + v->NPH - 1) / v->NPH;
        q.lds = sizeof(float4) * 2 * size_t(CPP) * G * q.IS;   // two phase buffers
        if (q.lds > 150 * 1024) continue;
        const int nbt_grid = ntile_n * NW;
        q.ws_bytes = size_t(nbt_grid) * q.NCG * TS * 64 * 16;
        p = q;
        return true;
    }
    return false;
}

hipError_t launch_pack_w_fwd_f32(const Geom &g, int NCG, int TS, int nblocks, const void *w,
                                 void *wf, size_t ws_bytes, hipStream_t s)
{
    const int total = nblocks * NCG * TS * 64;
    if (size_t(total) * 16 > ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_fwd_f32, dim3(std::min((total + 255) / 256, 1024)), dim3(256), 0, s,
                       (const float *)w, (float4 *)wf, g, NCG, TS, total);
    return hipGetLastError();
}

hipError_t launch_fwd_rf_f32(const Geom &g, const FwdBfPlan &p, const void *x, const void *w,
                             const void *bias, void *y, void *ws, int relu, hipStream_t s)
{
    const FwdRfVariant *v = pick_fwd_rf(p.NW, p.MB, p.TS, p.NCG, p.G * p.nblk);
    if (!v) return hipErrorInvalidValue;
    const int nbt_grid = (g.OC + 16 * p.NW - 1) / (16 * p.NW) * p.NW;
    const int total = nbt_grid * p.NCG * p.TS * 64;
    if (size_t(total) * 16 > p.ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_fwd_f32, dim3(std::min((total + 255) / 256, 1024)), dim3(256), 0, s,
                       (const float *)w, (float4 *)ws, g, p.NCG, p.TS, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    FwdRfArgs a{g, (const float *)x, (const float4 *)ws, (const float *)bias, (float *)y, relu,
                p.G, p.WP, p.IS, p.nblk};
    dim3 grid((g.B + p.G - 1) / p.G, (g.OC + 16 * p.NW - 1) / (16 * p.NW));
    e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
