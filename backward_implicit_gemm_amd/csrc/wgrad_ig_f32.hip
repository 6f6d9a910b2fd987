// wgrad_ig_f32.hip -- weight gradient on fp32 MFMA, split-K over images.
// Storage may be fp32 or bf16 (bf16 operands are widened exactly to fp32 as
// they are staged); the partials and their fixed-order sum are fp32.
//
// dW[oc][k] = sum_r dz[r][oc] * A[r][k] with r = (b,oh,ow), k = (ic,kh,kw):
// a GEMM with M = OC, N = IC*KH*KW and a reduction of B*OH*OW that is far
// longer than the output is wide, so the reduction is split across
// workgroups (grid.y) -- a few workgroups per output tile would leave most
// of the chip idle.  A workgroup owns a tile of BNK = 16*NBK columns of k and
// all OC rows (eight waves, two per SIMD: four split OC, two split the k
// tile), and a contiguous range of GS images that it
// walks in stages of G images: dz for the stage (masked by y > 0 under ReLU)
// is staged transposed ([oc][r]), and the x planes of the channels that the
// k tile touches are staged as contiguous NCHW slabs; both are double
// buffered, the next stage's loads in flight while the current one's MFMAs
// run.  The B operand
// is gathered from the slab through separable offsets (row part per r and
// column part per k, both held in registers for the whole kernel).  Each workgroup writes its
// fp32 partial tile; wgrad_reduce.hip sums the partials in fixed order.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

template <typename T>
struct WgradIgArgs {
    Geom g;
    const T *x, *dy, *ym;
    float *part;
    int relu;
    WgradIgPlan p;
    FastDiv fd_ocp;    // OC*P: dz elements per image
};

template <typename T, int NW, int MBW, int NBKW, int RS, int DV, int XV>
__global__ void __launch_bounds__(64 * NW) wgrad_ig_f32(WgradIgArgs<T> a)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const Geom &g = a.g;
    const WgradIgPlan &p = a.p;
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;   // oc group, k group of this wave
    constexpr int OCR = MBW * 64;   // oc rows covered by the four oc groups

    // Workgroups are dealt to the XCDs round-robin by id; ids are laid out so
    // that all column tiles of one split share an XCD and its L2, which then
    // serves that split's images of x and dy to every tile.
    const int xcd = int(blockIdx.x) % g.nxcd, slot = int(blockIdx.x) / g.nxcd;
    const int split = (slot / p.nkt) * g.nxcd + xcd;
    if (split >= p.splits) return;
    const int k0 = (slot % p.nkt) * p.BNK;
    const int bs = split * p.GS;
    const int be = min(g.B, bs + p.GS);
    const int ic_lo = k0 / g.KK;
    const int ic_hi = min(g.IC - 1, (min(k0 + p.BNK, g.K) - 1) / g.KK);
    const int nch = ic_hi - ic_lo + 1;

    float *dzt = lds;                               // [2][OCR][RP]
    float *xs = dzt + 2 * OCR * p.RP;               // [2][G][XSS]

    // zero both stage buffers once: padded rows / columns stay zero
    {
        const int n4 = (2 * OCR * p.RP + 2 * p.G * p.XSS) / 4;
        float4 *z = reinterpret_cast<float4 *>(lds);
        for (int i = tid; i < n4; i += NT) z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // row offsets into the slab of this lane's reduction slots r = 4*s +
    // lane/16 = (img, oh, ow) of a stage (0 for padding slots, whose dz is 0)
    int ro[RS];
#pragma unroll
    for (int s = 0; s < RS; ++s) {
        const int r = 4 * s + (lane >> 4);
        ro[s] = 0;
        if (r < p.G * g.P) {
            uint32_t img, pp, oh, ow;
            fdivmod(r, g.fd_P, img, pp);
            fdivmod(pp, g.fd_OW, oh, ow);
            ro[s] = int(img) * p.XSS + int(oh) * g.S * g.W + int(ow) * g.S;
        }
    }
    // column offsets of this lane's k columns into a slab image
    int koff[NBKW];
#pragma unroll
    for (int kb = 0; kb < NBKW; ++kb) {
        const int k = k0 + (wn * NBKW + kb) * 16 + (lane & 15);
        koff[kb] = 0;
        if (k < g.K) {
            uint32_t ic, t, kh, kw;
            fdivmod(k, g.fd_KK, ic, t);
            fdivmod(t, g.fd_KW, kh, kw);
            koff[kb] = (int(ic) - ic_lo) * g.HW + int(kh) * g.W + int(kw);
        }
    }

    // Stage staging through registers, fetched while the previous stage's
    // MFMAs run: dz (masked, then transposed into [oc][r] on the LDS write)
    // and the x planes of the channels this k tile touches (16-byte loads;
    // slot positions are fixed for the kernel, only the image base moves).
    float rd[DV];
    float4 rx[XV];
    const int xq_img = p.XSS >> 2;
    const int valid_x = nch * g.HW;
    int s_goff[XV], s_loff[XV], s_e[XV], s_img[XV];
#pragma unroll
    for (int j = 0; j < XV; ++j) {
        const int f = tid + j * NT;
        const int img = f / xq_img, e = (f % xq_img) * 4;
        s_img[j] = f < p.G * xq_img ? img : -1;
        s_e[j] = e;
        s_goff[j] = img * g.IC * g.HW + ic_lo * g.HW + e;
        s_loff[j] = img * p.XSS + e;
    }
    auto fetch = [&](int st) {
        const int b = bs + st * p.G;
        const int gimg = min(p.G, be - b);
        const int nd = gimg * g.OC * g.P;
        const size_t dbase = size_t(b) * g.OC * g.P;
#pragma unroll
        for (int j = 0; j < DV; ++j) {
            const int e = tid + j * NT;
            float v = 0.f;
            if (e < nd) {
                v = to_f32(a.dy[dbase + e]);
                if (a.relu && !(to_f32(a.ym[dbase + e]) > 0.f)) v = 0.f;
            }
            rd[j] = v;
        }
        const T *xbase = a.x + size_t(b) * g.IC * g.HW;
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            const int e = s_e[j];
            if (s_img[j] >= 0 && s_img[j] < gimg) {
                const T *src = xbase + s_goff[j];
                if (e + 3 < valid_x) {
                    v = ld4_f32(src);
                } else {
                    if (e + 0 < valid_x) v.x = to_f32(src[0]);
                    if (e + 1 < valid_x) v.y = to_f32(src[1]);
                    if (e + 2 < valid_x) v.z = to_f32(src[2]);
                }
            }
            rx[j] = v;
        }
    };
    auto stash = [&](int buf) {
        float *db = dzt + buf * OCR * p.RP;
#pragma unroll
        for (int j = 0; j < DV; ++j) {
            const int e = tid + j * NT;
            if (e < p.G * g.OC * g.P) {
                uint32_t img, rem, oc, pp;
                fdivmod(e, a.fd_ocp, img, rem);
                fdivmod(rem, g.fd_P, oc, pp);
                db[int(oc) * p.RP + int(img) * g.P + int(pp)] = rd[j];
            }
        }
        float *xb = xs + buf * p.G * p.XSS;
#pragma unroll
        for (int j = 0; j < XV; ++j)
            if (s_img[j] >= 0) *reinterpret_cast<float4 *>(xb + s_loff[j]) = rx[j];
    };

    f32x4 acc[MBW][NBKW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBKW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nst = be > bs ? (be - bs + p.G - 1) / p.G : 0;
    __syncthreads();                 // zero-fill done
    if (nst > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) fetch(st + 1);
        const float *db = dzt + buf * OCR * p.RP + (wm * MBW * 16 + (lane & 15)) * p.RP + (lane >> 4);
        const float *xb = xs + buf * p.G * p.XSS;
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const float *xr = xb + ro[s];
            float av[MBW], bv[NBKW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) av[mb] = db[mb * 16 * p.RP + s * 4];
#pragma unroll
            for (int kb = 0; kb < NBKW; ++kb) bv[kb] = xr[koff[kb]];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int kb = 0; kb < NBKW; ++kb)
                    acc[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mb], bv[kb], acc[mb][kb], 0, 0, 0);
        }
        if (st + 1 < nst) stash(buf ^ 1);
        __syncthreads();
    }

    float *out = a.part + size_t(split) * g.OC * g.K;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int oc = wm * MBW * 16 + mb * 16 + (lane >> 4) * 4 + v;
            if (oc >= g.OC) continue;
#pragma unroll
            for (int kb = 0; kb < NBKW; ++kb) {
                const int k = k0 + (wn * NBKW + kb) * 16 + (lane & 15);
                if (k < g.K) out[size_t(oc) * g.K + k] = acc[mb][kb][v];
            }
        }
}

template <typename T>
struct WgradVariant {
    int NW, MBW, NBKW, RS, DV, XV;
    void (*fn)(WgradIgArgs<T>);
};

#define WG_V(NW, MBW, NBKW, RS, DV, XV) \
    {NW, MBW, NBKW, RS, DV, XV, wgrad_ig_f32<T, NW, MBW, NBKW, RS, DV, XV>}
template <typename T>
const WgradVariant<T> kWgradVariants[] = {
    WG_V(8, 2, 6, 12, 12, 4),   // layers 1 and 2: 128 oc x 192 k, stages of 48 rows
    WG_V(8, 1, 6, 12, 12, 4), WG_V(8, 2, 2, 12, 12, 4), WG_V(8, 1, 2, 12, 12, 4),
};
#undef WG_V

int rup4(int v) { return (v + 3) / 4 * 4; }

template <typename T>
const WgradVariant<T> *pick_wgrad(int NW, int MBW, int NBK, int rs, int dv, int xv)
{
    for (const auto &v : kWgradVariants<T>)
        if (v.NW == NW && v.MBW == MBW && v.NBKW * (NW / 4) == NBK && v.RS == rs && dv <= v.DV &&
            xv <= v.XV)
            return &v;
    return nullptr;
}

}  // namespace

bool plan_wgrad_ig_f32(const Geom &g, WgradIgPlan &p)
{
    if (g.OC > 128 || g.P > 48) return false;
    const int MBW = g.OC <= 64 ? 1 : 2;
    const int RS = 12;                 // every variant reduces 48 rows per stage
    const size_t budget = 150 * 1024;
    for (int NBK : {12, 4}) {
        // stages of G images (at most 48 rows); fewer images when the x slab
        // would not fit the staging registers
        for (int G = std::max(1, std::min(g.B, 48 / g.P)); G >= 1; --G) {
            WgradIgPlan q;
            q.MBW = MBW; q.NBK = NBK; q.BNK = 16 * NBK;
            q.nkt = (g.K + q.BNK - 1) / q.BNK;
            q.NCHS = std::min(g.IC, (q.BNK - 1) / g.KK + 2);
            q.XSS = rup4(q.NCHS * g.HW);
            q.G = G;
            q.R4 = 4 * RS;
            q.RP = q.R4 + 2;           // = 2 mod 4: the 16 oc rows of an A read hit distinct banks
            q.NW = 8;
            q.DV = (q.G * g.OC * g.P + 64 * q.NW - 1) / (64 * q.NW);
            q.XV = (q.G * q.XSS / 4 + 64 * q.NW - 1) / (64 * q.NW);
            // split the batch so that tiles x splits covers the CUs once
            int splits = std::max(1, (g.ncu + q.nkt - 1) / q.nkt);
            const int max_splits = (g.B + q.G - 1) / q.G;
            splits = std::min(splits, max_splits);
            q.GS = ((g.B + splits - 1) / splits + q.G - 1) / q.G * q.G;
            q.splits = (g.B + q.GS - 1) / q.GS;
            q.lds = sizeof(float) * (2 * size_t(MBW * 64) * q.RP + 2 * size_t(q.G) * q.XSS);
            if (q.lds > budget) continue;
            if (!pick_wgrad<float>(q.NW, MBW, NBK, RS, q.DV, q.XV)) continue;
            p = q;
            return true;
        }
    }
    return false;
}

template <typename T>
hipError_t launch_wgrad_ig(const Geom &g, const WgradIgPlan &p, const void *x, const void *dy,
                           const void *ym, float *part, int relu, hipStream_t s)
{
    const WgradVariant<T> *v = pick_wgrad<T>(p.NW, p.MBW, p.NBK, p.R4 / 4, p.DV, p.XV);
    if (!v || 4 * v->RS != p.R4 || p.G * g.P > p.R4) return hipErrorInvalidValue;
    WgradIgArgs<T> a{g, (const T *)x, (const T *)dy, (const T *)ym, part, relu, p,
                     make_fastdiv(g.OC * g.P)};
    dim3 grid(g.nxcd * ((p.splits + g.nxcd - 1) / g.nxcd) * p.nkt);
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

template hipError_t launch_wgrad_ig<float>(const Geom &, const WgradIgPlan &, const void *,
                                           const void *, const void *, float *, int, hipStream_t);
template hipError_t launch_wgrad_ig<bf16_t>(const Geom &, const WgradIgPlan &, const void *,
                                            const void *, const void *, float *, int, hipStream_t);

}  // namespace gc
