// fwd_ws_f32.hip -- forward convolution, fp32 storage, fp32 MFMA
// (v_mfma_f32_16x16x4_f32), with loader waves and MFMA waves.
//
// The reduction runs in blocks of 16 k = 4 channels x 4 taps, so a lane's
// four MFMA steps read four consecutive channels at one tap: x staged
// channels-innermost [group][image][pixel][4] through 4x4 register
// transposes, weights pre-packed into float4 fragments and streamed from L2
// through a register ring.  When KH*KW = 4*(TS-1) + 1 (5x5 and 3x3 kernels),
// the last tap of each channel group is not padded to a step of its own:
// one step covers it for four groups, lane group q reading group 4l+q of
// the phase (FwdF32Steps), which removes the zero-padded taps' MFMAs.  The roles are split as in fwd_ws_bf16.hip, because a wave's
// vector-memory counter is in order and the x loads (HBM) would otherwise
// hold up every later weight-ring wait (L2):
//   * NWM loader waves: branch-free buffer loads (channels past IC and images
//     past the batch read zeros past the end of x; the last 4-pixel block of
//     a plane is moved back to end with it), register transposes, LDS stores;
//   * NWM MFMA waves, one 16-channel block each, A fragments read one tap step
//     ahead of their MFMAs.
// The fp32 x tile is too large for LDS at once, so the staging phases go
// through two buffers: in iteration ph the MFMA waves consume phase ph while
// the loaders store phase ph+1 (loaded during the previous iteration) into
// the other buffer and issue the loads of phase ph+2; one barrier per
// iteration hands the buffers over.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

struct FwdWsF32Args {
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

// GS: LDS slots per staged channel group, a compile-time bound on G*IS, so
// that the offsets of the groups and buffers are instruction immediates.
template <int NWM, int MB, int TS, int NCG, int CPP, int D, int GS, bool LO>
__global__ void __launch_bounds__(128 * NWM) __attribute__((amdgpu_waves_per_eu(1, NWM / 2)))
fwd_ws_f32(FwdWsF32Args a)
{
    extern __shared__ __attribute__((aligned(16))) float4 lds4f[];
    const Geom &g = a.g;
    constexpr FwdF32Steps ST{NCG, CPP, TS, LO};
    constexpr int NPH = ST.nph();
    constexpr int NFRAG = ST.nfrag();
    constexpr int TSF = ST.tsf();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b0 = blockIdx.x * a.G;
    const int gimg = min(a.G, g.B - b0);
    constexpr int gstride = GS;                     // float4 slots per channel group
    constexpr int bufsz = CPP * gstride;            // one phase buffer

    if (wave >= NWM) {
        // ---- loader waves: unit (channel group, image, 4-pixel block) ----
        const int lt = tid - 64 * NWM;
        const int units_per_cg = a.G * a.nblk;
        const int u_blk = lt % a.nblk, u_img = (lt / a.nblk) % a.G, u_cgl = lt / units_per_cg;
        const bool u_unit = u_cgl < CPP;
        const int u_w0 = min(4 * u_blk, g.HW - 4);
        const bool img_ok = u_img < gimg;
        const uint32_t plane = uint32_t(g.HW) * 4;
        const uint32_t u_off = (uint32_t(b0 + u_img) * g.IC * g.HW + u_w0) * 4;
        const __amdgpu_buffer_rsrc_t xrs = tensor_rsrc(a.x, uint32_t(g.B) * g.IC * plane);
        const int ih0 = u_w0 / g.W, iw0 = u_w0 - ih0 * g.W;
        float4 in[4];
        auto fetch = [&](int ph) {
            const int cg = ph * CPP + u_cgl;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int ic = cg * 4 + c;
                const bool ok = u_unit && cg < NCG && img_ok && ic < g.IC;
                in[c] = bload16(xrs, ok ? u_off + uint32_t(ic) * plane : kOffNone);
            }
        };
        auto stash = [&](int ph) {
            const int cg = ph * CPP + u_cgl;
            if (!u_unit || cg >= NCG) return;
            float4 *dst = lds4f + (ph & 1) * bufsz + u_cgl * gstride + u_img * a.IS;
            int ih = ih0, iw = iw0;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                dst[ih * a.WP + iw] = make_float4(comp(in[0], pp), comp(in[1], pp), comp(in[2], pp),
                                                  comp(in[3], pp));
                if (++iw == g.W) { iw = 0; ++ih; }
            }
        };
        fetch(0);
        stash(0);
        if (NPH > 1) fetch(1);
        __syncthreads();
        for (int ph = 0; ph < NPH; ++ph) {
            if (ph + 1 < NPH) {
                stash(ph + 1);
                if (ph + 2 < NPH) fetch(ph + 2);
            }
            __syncthreads();
        }
        return;
    }

    // ---- MFMA waves: one 16-channel block each ----
    const int nb = blockIdx.y * NWM + wave;
    // fragment f of this wave's block: byte offset w_vo + f*1024 of the packed
    // weights (the per-fragment part is a constant, so no address registers)
    const __amdgpu_buffer_rsrc_t wrs = tensor_rsrc(a.wf, uint32_t(gridDim.y) * NWM * NFRAG * 1024);
    const uint32_t w_vo = (uint32_t(nb) * NFRAG * 64 + lane) * 16;
    float4 ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        ring[i] = i < NFRAG ? bload16s(wrs, w_vo, i * 1024) : make_float4(0.f, 0.f, 0.f, 0.f);

    const int rows = gimg * g.P;
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
    int toff[TSF];
#pragma unroll
    for (int s = 0; s < TSF; ++s) {
        const int t = 4 * s + (lane >> 4);
        toff[s] = 0;
        if (t < g.KK) {
            uint32_t kh, kw;
            fdivmod(t, g.fd_KW, kh, kw);
            toff[s] = int(kh) * a.WP + int(kw);
        }
    }
    // shared steps: the last tap, in channel group (4l + q) of the phase
    int t_last = 0, q_last = 0;
    if (LO) {
        uint32_t kh, kw;
        fdivmod(uint32_t(g.KK - 1), g.fd_KW, kh, kw);
        t_last = int(kh) * a.WP + int(kw);
        q_last = (lane >> 4) * gstride + t_last;
    }

    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS slot of step k's A operand for row block mb (phase-relative): a full
    // step (group k / TSF, taps 4*(k % TSF) + q) or shared step l = k - nfull
    // (lanes past the phase's groups read a valid slot; their B is zero)
    auto a_slot = [&](int ph, int k, int mb) {
        const int nfull = ST.nfull(ph);
        if (k < nfull) return (k / TSF) * gstride + rowoff[mb] + toff[k % TSF];
        const int l = k - nfull;
        const int nv = ST.ncg(ph) - 4 * l;
        return 4 * l * gstride + rowoff[mb] + ((lane >> 4) < nv ? q_last : t_last);
    };

    __syncthreads();                                 // phase 0 staged
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        const float4 *xbuf = lds4f + (ph & 1) * bufsz;
        const int nst = ST.nsteps(ph), f0 = ST.base(ph);
        // A fragments one step ahead of their MFMAs
        float4 af[2][MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[0][mb] = xbuf[a_slot(ph, 0, mb)];
#pragma unroll
        for (int k = 0; k < nst; ++k) {
            const int f = f0 + k;
            const int cur = k & 1;
            if (k + 1 < nst) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) af[cur ^ 1][mb] = xbuf[a_slot(ph, k + 1, mb)];
            }
            const float4 bv = ring[f % D];
            if (f + D < NFRAG) ring[f % D] = bload16s(wrs, w_vo, (f + D) * 1024);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(af[cur][mb], j), comp(bv, j),
                                                                   acc[mb], 0, 0, 0);
            // keep each step's loads in their place: hoisting later steps'
            // loads above these MFMAs would only lengthen register lives
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();                             // phase ph done, ph+1 staged
    }

    // epilogue: row r = mb*16 + 4*(lane/16) + v, column nb*16 + lane%16
    const int n = nb * 16 + (lane & 15);
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

struct FwdWsF32Variant {
    int NWM, MB, TS, NCG, CPP, GS;
    void (*fn[2])(FwdWsF32Args);     // [shared last-tap steps]
};
#define WF_V(NWM, MB, TS, NCG, CPP, GS)                                   \
    {NWM, MB, TS, NCG, CPP, GS,                                           \
     {fwd_ws_f32<NWM, MB, TS, NCG, CPP, 8, GS, false>,                    \
      fwd_ws_f32<NWM, MB, TS, NCG, CPP, 8, GS, true>}}
const FwdWsF32Variant kFwdWsF32Variants[] = {
    // 59 -> 128, 11x15, 5x5, stride 3 (12 rows per image), 128 channels per workgroup
    WF_V(8, 3, 7, 15, 3, 960),    // 3 or 4 images, 36 or 48 rows
    WF_V(8, 2, 7, 15, 6, 480),    // 2 images
    WF_V(8, 1, 7, 15, 12, 240),   // one image
    // 128 -> 128, 3x4, 3x3 (2 rows per image), 64 channels per workgroup
    WF_V(4, 4, 3, 32, 2, 512),    // 32 images
    WF_V(4, 2, 3, 32, 5, 256),    // 16 images
    WF_V(4, 1, 3, 32, 10, 128),   // 8 images
    WF_V(4, 1, 3, 32, 21, 64),    // 4 images
    WF_V(4, 1, 3, 32, 32, 32),    // one or two images
};
#undef WF_V

const FwdWsF32Variant *pick_fwd_ws_f32(int NWM, int MB, int TS, int NCG, int CPP, int gslots)
{
    for (const auto &v : kFwdWsF32Variants)
        if (v.NWM == NWM && v.MB == MB && v.TS == TS && v.NCG == NCG && v.CPP == CPP && gslots <= v.GS)
            return &v;
    return nullptr;
}

}  // namespace

// NWM = 8 MFMA waves (128 channels per workgroup) for layer-1-like shapes, 4
// (64 channels, twice the column tiles) where an image has 4 rows or fewer;
// then, over the G (images per workgroup) that have an instantiation, the one
// that (1) puts the most workgroups on the chip at once, up to one per CU,
// (2) wastes the fewest MFMA rows, (3) is larger (fewer passes of the weight
// stream per image).  CPP: the channel groups the loader threads stage per
// phase.
bool plan_fwd_ws_f32(const Geom &g, FwdWsPlan &p)
{
    if (g.P > 64 || g.KK > 36 || g.HW < 4) return false;
    if (size_t(g.B) * g.IC * g.HW * 4 >= (size_t(1) << 31)) return false;
    // the weight packing runs one grid row per 16-channel block (at most 65535)
    if ((g.OC + 15) / 16 > 65535) return false;
    const int NWM = g.P <= 4 ? 4 : 8;
    const int TS = (g.KK + 3) / 4, NCG = (g.IC + 3) / 4, nblk = (g.HW + 3) / 4;
    const int ntile = (g.OC + 16 * NWM - 1) / (16 * NWM);
    const int loaders = 64 * NWM;
    bool found = false;
    int best_wgs = 0, best_g = 0;
    double best_fill = 0.0;
    for (int G = std::min(g.B, std::max(1, 64 / g.P)); G >= 1; --G) {
        FwdWsPlan q{};
        q.NWM = NWM; q.NBW = 1; q.TS = TS; q.NCG = NCG; q.nblk = nblk; q.ntile = ntile; q.G = G;
        q.MB = (G * g.P + 15) / 16;
        const int units_per_cg = G * nblk;
        if (units_per_cg > loaders) continue;
        const long long groups = (g.B + G - 1) / G;
        const int wgs = int(std::min<long long>(groups * ntile, g.ncu));
        const double fill = double(G * g.P) / (16.0 * q.MB);
        const bool better = !found || wgs > best_wgs ||
                            (wgs == best_wgs && (fill > best_fill + 1e-9 ||
                                                 (fill > best_fill - 1e-9 && G > best_g)));
        if (!better) continue;
        pick_lds_pitch(g, G, q.MB, TS, q.WP, q.IS);
        // as many channel groups per phase as the loaders can stage, or
        // fewer where only that has an instantiation
        const FwdWsF32Variant *v = nullptr;
        for (q.CPP = std::min(NCG, loaders / units_per_cg); q.CPP >= 1 && !v; --q.CPP)
            v = pick_fwd_ws_f32(NWM, q.MB, TS, NCG, q.CPP, G * q.IS);
        ++q.CPP;
        if (!v) continue;
        q.lds = sizeof(float4) * 2 * size_t(q.CPP) * v->GS;
        if (q.lds > 150 * 1024) continue;
        q.lo = TS >= 2 && g.KK == 4 * (TS - 1) + 1;
        q.ws_bytes = size_t(ntile) * NWM * FwdF32Steps{NCG, q.CPP, TS, q.lo}.nfrag() * 64 * 16;
        p = q;
        found = true;
        best_wgs = wgs; best_fill = fill; best_g = G;
    }
    return found;
}

hipError_t launch_fwd_ws_f32(const Geom &g, const FwdWsPlan &p, const void *x, const void *w,
                             const void *bias, void *y, void *ws, int relu, hipStream_t s)
{
    const FwdWsF32Variant *v = pick_fwd_ws_f32(p.NWM, p.MB, p.TS, p.NCG, p.CPP, p.G * p.IS);
    if (!v || p.G * p.nblk * p.CPP > 64 * p.NWM || g.HW < 4 || p.G * g.P > 16 * p.MB ||
        p.lds < sizeof(float4) * 2 * size_t(p.CPP) * v->GS)
        return hipErrorInvalidValue;
    if (p.lo && !(p.TS >= 2 && g.KK == 4 * (p.TS - 1) + 1)) return hipErrorInvalidValue;
    void (*fn)(FwdWsF32Args) = v->fn[p.lo ? 1 : 0];
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(fn));
    if (e != hipSuccess) return e;
    e = launch_pack_w_fwd_f32(g, p.NCG, p.CPP, p.TS, p.lo, p.ntile * p.NWM, w, ws, p.ws_bytes, s);
    if (e != hipSuccess) return e;
    FwdWsF32Args a{g, (const float *)x, (const float4 *)ws, (const float *)bias, (float *)y, relu,
                   p.G, p.WP, p.IS, p.nblk};
    hipLaunchKernelGGL(fn, dim3((g.B + p.G - 1) / p.G, p.ntile), dim3(128 * p.NWM), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
