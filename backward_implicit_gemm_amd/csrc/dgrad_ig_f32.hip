// dgrad_ig_f32.hip -- d_input on fp32 MFMA, image-group tiling, gather form.
// Storage may be fp32 or bf16: bf16 operands are widened exactly to fp32 as
// they are staged into LDS, and the result is rounded to bf16 once, on store.
//
// For a group of G whole images the workgroup first forms, chunk by chunk of
// CC input channels, the column gradient
//     dcol[(b,oh,ow)][(icl,kh,kw)] = sum_oc dz[b,oc,oh,ow] * w[oc, c0+icl, kh, kw]
// as an MFMA GEMM (M = G*OH*OW rows, N = CC*KH*KW, reduction over OC in
// sub-chunks of OCS channels, v_mfma_f32_16x16x4_f32), with dz = dy masked by
// (y > 0) when the layer has a ReLU, staged once per workgroup.  Weight
// sub-chunks are fetched with 16-byte loads while the previous sub-chunk's
// MFMAs run and written to the other half of a double-buffered LDS; the NW
// waves (two per SIMD on the policy-network layers) split the dcol columns.
// The dcol tile goes to LDS, and every input-gradient element of the chunk is
// then gathered from it:
//     dx[b,ic,ih,iw] = sum over the (oh,kh) with oh*S + kh = ih and the
//                      (ow,kw) with ow*S + kw = iw of dcol[...]
// using the dcol offsets of each pixel's taps, computed once per thread.  Each
// dx element is written exactly once (uncovered pixels get an empty sum, 0),
// so there are no atomics and no zero-fill pass.  The MACs are the
// algorithmic ones: only taps that land on an output position are multiplied.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

template <typename T>
struct DgradIgArgs {
    Geom g;
    const T *dy, *w, *ym;
    T *dx;
    int relu;
    DgradIgPlan p;
    FastDiv fd_ocp;    // OC*P: dz elements per image
    FastDiv fd_cc;     // CC: chunk planes per image
    FastDiv fd_nq;     // ceil(NCH/4): float4 slots per weight row
};

template <typename T, int NW, int MB, int NBW, int KSD, int TAPS, int WV>
__global__ void __launch_bounds__(64 * NW) dgrad_ig_f32(DgradIgArgs<T> a)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const Geom &g = a.g;
    const DgradIgPlan &p = a.p;
    constexpr int NT = 64 * NW;
    constexpr int RM = MB * 16;
    constexpr int OCS = 4 * KSD;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const int b0 = blockIdx.x * p.G;
    const int gimg = min(p.G, g.B - b0);
    const int ch_begin = blockIdx.y * p.cpg;
    const int ch_end = min(ch_begin + p.cpg, p.nchunks);

    float *dz = lds;                               // [RM][DZP]
    float *wc = dz + RM * p.DZP;                   // [2][OCS][WCP]
    float *dcol = wc + 2 * OCS * p.WCP;            // [RM][DCP]
    const int nq = (p.NCH + 3) >> 2;               // float4 slots per weight row

    // dz must be zero in padding rows/columns; weight columns past the
    // staged float4 slots (4*nq <= k < 16*NBT) must read as 0.
    {
        const int n4 = RM * p.DZP / 4;
        float4 *z = reinterpret_cast<float4 *>(dz);
        for (int i = tid; i < n4; i += NT) z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int pad = 16 * p.NBT - 4 * nq;
        for (int i = tid; i < 2 * OCS * pad; i += NT) {
            const int row = i / pad, k = 4 * nq + i % pad;
            wc[row * p.WCP + k] = 0.f;
        }
    }

    // This thread gathers input pixel q = (ih, iw) of planes r0, r0+rpi, ...
    // of each chunk (a plane is one (image, channel) pair).  Pixel (ih, iw)
    // receives dcol[(oh,ow)][(kh,kw)] for every oh*S + kh = ih, ow*S + kw = iw;
    // the dcol offsets of those taps are fixed for the whole kernel.
    const int rpi = NT / g.HW;
    const bool gather = tid < rpi * g.HW;
    const int q = gather ? tid % g.HW : 0;
    const int r0 = gather ? tid / g.HW : 0;
    int toff[TAPS];
    int ntap = 0;
    {
        const int ih = q / g.W, iw = q % g.W;
#pragma unroll
        for (int j = 0; j < TAPS; ++j) toff[j] = 0;
        for (int oh = 0; oh < g.OH; ++oh) {
            const int kh = ih - oh * g.S;
            if (kh < 0 || kh >= g.KH) continue;
            for (int ow = 0; ow < g.OW; ++ow) {
                const int kw = iw - ow * g.S;
                if (kw < 0 || kw >= g.KW) continue;
                const int off = (oh * g.OW + ow) * p.DCP + kh * g.KW + kw;
#pragma unroll
                for (int j = 0; j < TAPS; ++j)
                    if (j == ntap) toff[j] = off;
                ++ntap;
            }
        }
    }
    __syncthreads();

    // dz rows (b,oh,ow) x columns oc, masked by the forward output
    {
        const int n = gimg * g.OC * g.P;
        const size_t base = size_t(b0) * g.OC * g.P;
        for (int e = tid; e < n; e += NT) {
            uint32_t img, rem, oc, pp;
            fdivmod(e, a.fd_ocp, img, rem);
            fdivmod(rem, g.fd_P, oc, pp);
            float v = to_f32(a.dy[base + e]);
            if (a.relu && !(to_f32(a.ym[base + e]) > 0.f)) v = 0.f;
            dz[(int(img) * g.P + int(pp)) * p.DZP + int(oc)] = v;
        }
    }

    // Staging slots of this thread in a weight sub-chunk: slot j covers
    // float4 f = tid + NT*j = (row ocl, k offset 4*qq); fixed for the kernel.
    int s_goff[WV], s_loff[WV], s_kl[WV], s_row[WV];
#pragma unroll
    for (int j = 0; j < WV; ++j) {
        const int f = tid + j * NT;
        uint32_t ocl, qq;
        fdivmod(f, a.fd_nq, ocl, qq);
        s_row[j] = f < OCS * nq ? int(ocl) : -1;
        s_kl[j] = int(qq) * 4;
        s_goff[j] = int(ocl) * g.K + s_kl[j];
        s_loff[j] = int(ocl) * p.WCP + s_kl[j];
    }
    float4 rw[WV];
    auto fetch = [&](int st) {
        const int ch = ch_begin + st / p.nsub, sub = st % p.nsub;
        const int c0 = ch * p.CC, oc0 = sub * OCS;
        const int valid_k = min(p.CC, g.IC - c0) * g.KK;
        const T *base = a.w + size_t(oc0) * g.K + size_t(c0) * g.KK;
#pragma unroll
        for (int j = 0; j < WV; ++j) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            const int kl = s_kl[j];
            if (s_row[j] >= 0 && oc0 + s_row[j] < g.OC) {
                const T *src = base + s_goff[j];
                if (kl + 3 < valid_k) {
                    v = ld4_f32(src);
                } else {
                    if (kl + 0 < valid_k) v.x = to_f32(src[0]);
                    if (kl + 1 < valid_k) v.y = to_f32(src[1]);
                    if (kl + 2 < valid_k) v.z = to_f32(src[2]);
                }
            }
            rw[j] = v;
        }
    };
    auto stash = [&](int buf) {
        float *wb = wc + buf * OCS * p.WCP;
#pragma unroll
        for (int j = 0; j < WV; ++j)
            if (s_row[j] >= 0) *reinterpret_cast<float4 *>(wb + s_loff[j]) = rw[j];
    };

    f32x4 acc[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nst = (ch_end - ch_begin) * p.nsub;
    if (nst > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        const int sub = st % p.nsub;
        if (st + 1 < nst) fetch(st + 1);
        const float *wb = wc + buf * OCS * p.WCP + (lane >> 4) * p.WCP + (lane & 15);
        const float *ab = dz + (lane & 15) * p.DZP + sub * OCS + (lane >> 4);
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            float av[MB], bv[NBW];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) av[mb] = ab[mb * 16 * p.DZP + s * 4];
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nbg = wave + NW * j;
                bv[j] = nbg < p.NBT ? wb[s * 4 * p.WCP + nbg * 16] : 0.f;
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int j = 0; j < NBW; ++j)
                    acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mb], bv[j], acc[mb][j], 0, 0, 0);
        }
        if (st + 1 < nst) stash(buf ^ 1);
        if (sub == p.nsub - 1) {
            // dcol tile of this chunk -> LDS
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const int nbg = wave + NW * j;
                    if (nbg < p.NBT) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            dcol[(mb * 16 + (lane >> 4) * 4 + v) * p.DCP + nbg * 16 + (lane & 15)] = acc[mb][j][v];
                    }
                    acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            __syncthreads();
            // gather every dx element of the chunk from dcol
            const int ch = ch_begin + st / p.nsub;
            const int c0 = ch * p.CC;
            const int cc = min(p.CC, g.IC - c0);
            if (gather) {
                for (int row = r0; row < gimg * p.CC; row += rpi) {
                    uint32_t img, icl;
                    fdivmod(row, a.fd_cc, img, icl);
                    if (int(icl) >= cc) continue;
                    const float *dc = dcol + int(img) * g.P * p.DCP + int(icl) * g.KK;
                    float sum = 0.f;
#pragma unroll
                    for (int j = 0; j < TAPS; ++j)
                        if (j < ntap) sum += dc[toff[j]];
                    a.dx[(size_t(b0) + img) * g.IC * g.HW + size_t(c0 + int(icl)) * g.HW + q] =
                        from_f32<T>(sum);
                }
            }
        }
        __syncthreads();
    }
}

template <typename T>
struct DgradVariant {
    int NW, MB, NBW, KSD, TAPS, WV;
    void (*fn)(DgradIgArgs<T>);
};

#define DG_V(NW, MB, NBW, KSD, TAPS, WV) \
    {NW, MB, NBW, KSD, TAPS, WV, dgrad_ig_f32<T, NW, MB, NBW, KSD, TAPS, WV>}
template <typename T>
const DgradVariant<T> kDgradVariants[] = {
    DG_V(8, 3, 1, 16, 4, 4),    // layer 1: 4 images x 12 rows, 5 channels x 25 taps, 2x2 taps/pixel
    DG_V(4, 4, 1, 16, 9, 4),    // layer 2: 32 images x 2 rows, 7 channels x 9 taps, 3x3 taps/pixel
    DG_V(4, 1, 1, 16, 9, 4), DG_V(4, 2, 1, 16, 9, 4), DG_V(4, 3, 1, 16, 9, 4),
    DG_V(4, 1, 1, 16, 16, 8), DG_V(4, 2, 1, 16, 16, 8), DG_V(4, 3, 1, 16, 16, 8),
    DG_V(4, 4, 1, 16, 16, 8),
    DG_V(4, 1, 2, 16, 16, 8), DG_V(4, 2, 2, 16, 16, 8), DG_V(4, 3, 2, 16, 16, 8),
    DG_V(4, 4, 2, 16, 16, 8),
    DG_V(8, 1, 1, 16, 16, 4), DG_V(8, 2, 1, 16, 16, 4), DG_V(8, 3, 1, 16, 16, 4),
    DG_V(8, 4, 1, 16, 16, 4),
    DG_V(4, 1, 1, 16, 36, 8), DG_V(4, 2, 2, 16, 36, 8),
};
#undef DG_V

int rup(int v, int m) { return (v + m - 1) / m * m; }

template <typename T>
const DgradVariant<T> *pick_dgrad(int NW, int MB, int NBW, int taps, int wv)
{
    const DgradVariant<T> *best = nullptr;
    for (const auto &v : kDgradVariants<T>)
        if (v.NW == NW && v.MB == MB && v.NBW == NBW && taps <= v.TAPS && wv <= v.WV &&
            (!best || v.TAPS < best->TAPS || (v.TAPS == best->TAPS && v.WV < best->WV)))
            best = &v;
    return best;
}

// smallest stride >= n with stride % 32 == r
int stride_mod32(int n, int r) { return n + ((r - n % 32) % 32 + 32) % 32; }

}  // namespace

bool plan_dgrad_ig_f32(const Geom &g, DgradIgPlan &p)
{
    if (g.P > 64 || g.HW > 256) return false;
    int G = 64 / g.P;
    if (G > g.B) G = g.B;
    if (g.P == 12 && G > 4) G = 4;
    const int MB = (G * g.P + 15) / 16;
    const int ngroups = (g.B + G - 1) / G;
    const int TH = (g.KH + g.S - 1) / g.S, TW = (g.KW + g.S - 1) / g.S;
    const int OCS = 64;   // every variant reduces over 16 MFMA steps of 4 channels
    const size_t budget = 150 * 1024;

    bool found = false;
    double best = -1.0;
    for (int NW : {8, 4}) {
        for (int CC = 1; CC <= std::min(g.IC, 32); ++CC) {
            DgradIgPlan q;
            q.NW = NW; q.G = G; q.MB = MB; q.CC = CC;
            q.NCH = CC * g.KK;
            q.NBT = (q.NCH + 15) / 16;
            q.NBW = (q.NBT + NW - 1) / NW;
            if (q.NBW > 2) break;
            q.OCS = OCS;
            q.nsub = (g.OC + OCS - 1) / OCS;
            q.OCP = q.nsub * OCS;
            q.DZP = q.OCP + 2;
            q.WCP = stride_mod32(q.NBT * 16, 16);
            q.DCP = stride_mod32(q.NBT * 16, 16);
            q.TH = TH; q.TW = TW;
            q.nchunks = (g.IC + CC - 1) / CC;
            q.cgroups = 1;
            while (ngroups * q.cgroups < g.ncu && q.cgroups * 2 <= q.nchunks) q.cgroups *= 2;
            q.cpg = (q.nchunks + q.cgroups - 1) / q.cgroups;
            q.cgroups = (q.nchunks + q.cpg - 1) / q.cpg;
            q.WV = (OCS * ((q.NCH + 3) / 4) + 64 * NW - 1) / (64 * NW);
            q.lds = sizeof(float) * (size_t(16 * MB) * q.DZP + 2 * size_t(OCS) * q.WCP +
                                     size_t(16 * MB) * q.DCP);
            if (q.lds > budget) continue;
            if (!pick_dgrad<float>(NW, MB, q.NBW, TH * TW, q.WV)) continue;
            // MFMA slots used: dcol columns over the columns the waves compute
            const double eff = double(q.NCH) / (q.NBW * NW * 16);
            if (eff > best + 1e-9) {
                best = eff;
                p = q;
                found = true;
            }
        }
        // eight waves only when they keep the MFMAs well used
        if (found && best >= 0.9) break;
    }
    return found;
}

template <typename T>
hipError_t launch_dgrad_ig(const Geom &g, const DgradIgPlan &p, const void *dy, const void *w,
                           const void *ym, void *dx, int relu, hipStream_t s)
{
    const DgradVariant<T> *v = pick_dgrad<T>(p.NW, p.MB, p.NBW, p.TH * p.TW, p.WV);
    if (!v || 4 * v->KSD != p.OCS || g.HW > 64 * p.NW) return hipErrorInvalidValue;
    DgradIgArgs<T> a{g, (const T *)dy, (const T *)w, (const T *)ym, (T *)dx, relu, p,
                     make_fastdiv(g.OC * g.P), make_fastdiv(p.CC), make_fastdiv((p.NCH + 3) / 4)};
    dim3 grid((g.B + p.G - 1) / p.G, p.cgroups);
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

template hipError_t launch_dgrad_ig<float>(const Geom &, const DgradIgPlan &, const void *,
                                           const void *, const void *, void *, int, hipStream_t);
template hipError_t launch_dgrad_ig<bf16_t>(const Geom &, const DgradIgPlan &, const void *,
                                            const void *, const void *, void *, int, hipStream_t);

}  // namespace gc
