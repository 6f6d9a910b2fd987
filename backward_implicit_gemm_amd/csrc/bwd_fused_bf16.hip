// bwd_fused_bf16.hip -- the bf16 backward (d_input and wgrad) in three or
// four launches instead of five.
//
// The separate calls launch: the d_input weight packing, the d_input kernel,
// the dz regrouping, the wgrad partial-tile kernel and the fixed-order
// reduction.  Here:
//   1. one pre-pass launch: the first ngroups*kDzSlices workgroups regroup dz (masked) for
//      wgrad, the rest pack the weights for d_input;
//   2. one main launch whose grid holds the d_input workgroups followed by the
//      wgrad workgroups -- the two sets are independent, so they run side by
//      side and neither waits for the other's tail -- when that costs the
//      d_input kernel no occupancy that matters (see the planner), else the
//      two main kernels one after the other;
//   3. the fixed-order reduction of the wgrad partials.
// Both main bodies are the ones the separate calls run, so dx and dw are
// bit-identical to gc_conv_bwd_data + gc_conv_bwd_weight.  The reduction
// stays a launch of its own: folding it into the main launch would need one
// workgroup to wait for others, and the partial tiles are summed in split
// order so the result does not depend on scheduling.
#include "dgrad_ig_bf16_dev.h"
#include "wgrad_ig_bf16_dev.h"

namespace gc {
namespace {

__global__ void __launch_bounds__(kDzNT) bwd_prep_bf16(const u16 *__restrict__ dy,
                                                       const u16 *__restrict__ ym,
                                                       uint4 *__restrict__ dzg, Geom g, int relu,
                                                       int PP, int ngroups,
                                                       const u16 *__restrict__ w,
                                                       uint4 *__restrict__ wp, int CC,
                                                       FastDiv fd_nbc, FastDiv fd_ks, int total,
                                                       int npack)
{
    const int bid = blockIdx.x;
    if (bid < ngroups * kDzSlices)
        dz_groups_bf16_body(dy, ym, dzg, g, relu, PP, bid);
    else
        pack_w_dgrad_bf16_body(w, wp, g, CC, fd_nbc, fd_ks, total, bid - ngroups * kDzSlices, npack);
}

// d_input workgroups first (n_dg of them, an (image group, channel group)
// grid of nx_dg columns, padded to a multiple of the XCD count), then the wgrad
// workgroups; the padding keeps each wgrad workgroup on the XCD its own
// decode expects (workgroup ids go round-robin over the XCDs).
template <int NW, int MB, int KS, int TAPS, int NBW, int GP, int NSTEP>
__global__ void __launch_bounds__(64 * NW) bwd_fused_bf16(DgradBfArgs da, WgradBfArgs wa, int n_dg,
                                                          int nx_dg, int n_dg_pad)
{
    const int bid = blockIdx.x;
    if (bid < n_dg)
        dgrad_ig_bf16_body<NW, MB, KS, TAPS, NBW, GP>(da, bid % nx_dg, bid / nx_dg);
    else if (bid >= n_dg_pad)
        wgrad_ig_bf16_body<NSTEP>(wa, bid - n_dg_pad);
}

struct FusedVariant {
    int MB, KS, TAPS, NBW, NSTEP, JW;
    void (*fn)(DgradBfArgs, WgradBfArgs, int, int, int);   // both grids in one launch
    void (*fn_d)(DgradBfArgs);                              // d_input alone
    void (*fn_w)(WgradBfArgs);                              // wgrad alone (16 waves)
};
// The (d_input, wgrad) kernel pairs the planners choose for the policy
// network's layers at B=1024 and B=16384; other shapes use separate calls.
#define FV(MB, KS, TAPS, NBW, NSTEP, JW)                                              \
    {MB, KS, TAPS, NBW, NSTEP, JW, bwd_fused_bf16<8, MB, KS, TAPS, NBW, 2, NSTEP>,     \
     dgrad_ig_bf16<8, MB, KS, TAPS, NBW, 2>, wgrad_ws_bf16<NSTEP, JW, false>}
// (both grids in one launch run the 8-wave wgrad body, whose tiles are 128
// columns: JW = 2)
const FusedVariant kFusedVariants[] = {
    FV(3, 4, 4, 1, 3, 2), FV(3, 4, 4, 1, 3, 4),    // 59 -> 128, 11x15, 5x5, stride 3
    FV(3, 4, 2, 1, 1, 2), FV(3, 4, 2, 1, 1, 4),    // 128 -> 128, 3x4, 3x3, B=1024
    FV(2, 4, 2, 2, 1, 2), FV(2, 4, 2, 2, 1, 4),    // 128 -> 128, 3x4, 3x3, B=16384
};
#undef FV

const FusedVariant *pick_fused(const DgradBfPlan &d, const WgradBfPlan &w)
{
    if (d.NW != 8 || d.GP != 2) return nullptr;
    for (const auto &v : kFusedVariants)
        if (v.MB == d.MB && v.KS == d.KS && v.TAPS == d.TAPS && v.NBW == d.NBW &&
            v.NSTEP == w.NSTEP && v.JW == w.JW)
            return &v;
    return nullptr;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

bool plan_bwd_fused_bf16(const Geom &g, BwdFusedBfPlan &p)
{
    BwdFusedBfPlan q{};
    if (!plan_dgrad_ig_bf16(g, q.d) || !plan_wgrad_ig_bf16(g, q.w)) return false;
    // One grid for both main kernels gives every workgroup the larger LDS
    // size, which can cut how many d_input workgroups share a CU.  Put them
    // in one launch only when the d_input grid still fits the chip in one
    // round at that size (the small problems, where the saved launch and
    // the overlap of the two tails matter); else launch them one after the
    // other, keeping the merged pre-pass.
    // The single grid runs the 8-wave wgrad body, whose tiles are 128 columns
    WgradBfPlan w128{};
    const bool have128 = plan_wgrad_bf16_tiles(g, 2, w128);
    const size_t lds = have128 ? std::max(q.d.lds, w128.lds) : 0;
    const int per_cu = lds ? int((160 * 1024) / lds) : 8;
    const int n_dg = (g.B + q.d.G - 1) / q.d.G * q.d.cgroups;
    q.fuse_main = have128 && n_dg <= g.ncu * std::max(per_cu, 1);
    if (q.fuse_main) q.w = w128;
    if (!pick_fused(q.d, q.w)) return false;
    q.ws_w_offset = align256(q.d.ws_bytes);
    q.ws_bytes = q.ws_w_offset + q.w.ws_bytes;
    p = q;
    return true;
}

hipError_t launch_bwd_fused_bf16(const Geom &g, const BwdFusedBfPlan &p, const void *x,
                                 const void *w, const void *dy, const void *ym, void *dx, void *dw,
                                 void *ws, int relu, hipStream_t s)
{
    const DgradBfPlan &d = p.d;
    const WgradBfPlan &wp = p.w;
    const FusedVariant *v = pick_fused(d, wp);
    if (!v) return hipErrorInvalidValue;
    // the preconditions of the two kernels, as their own launches check them
    if (g.HW > 64 * d.NW || d.G % 4 || d.G * g.P > 16 * d.MB || d.NBC > d.NW * d.NBW ||
        d.RP < 16 * d.MB + d.G || d.CC * (d.G / 4) > d.GP * ((64 * d.NW) / g.HW))
        return hipErrorInvalidValue;
    if (2 * wp.CCW * wp.nblk > kWgNT || wp.PP * 128 != wp.NSTEP * kWgNT || g.OC > 128 || g.HW < 8 ||
        kDzOC * g.P > kDzChunks * kDzNT || (p.fuse_main && wp.JW != 2))
        return hipErrorInvalidValue;
    const int total = d.nchunks * d.NBC * d.KS * 64;
    if (size_t(total) * 16 > d.ws_bytes) return hipErrorInvalidValue;
    if (reinterpret_cast<uintptr_t>(ws) % 256) return hipErrorInvalidValue;

    uint4 *wpk = static_cast<uint4 *>(ws);
    char *wsw = static_cast<char *>(ws) + p.ws_w_offset;
    uint4 *dzg = reinterpret_cast<uint4 *>(wsw);
    float *part = reinterpret_cast<float *>(wsw + wp.dz_bytes);

    // 1. dz regrouping and d_input weight packing
    const int npack = std::min((total + 255) / 256, 2048);
    const size_t dz_lds = dz_groups_lds(g);
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(&bwd_prep_bf16));
    if (e == hipSuccess) e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e == hipSuccess) e = allow_max_lds(reinterpret_cast<const void *>(v->fn_d));
    if (e == hipSuccess) e = allow_max_lds(reinterpret_cast<const void *>(v->fn_w));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_prep_bf16, dim3(wp.ngroups * kDzSlices + npack), dim3(kDzNT), dz_lds, s,
                       (const u16 *)dy, (const u16 *)ym, dzg, g, relu, wp.PP, wp.ngroups,
                       (const u16 *)w, wpk, d.CC, make_fastdiv(d.NBC), make_fastdiv(d.KS), total, npack);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2. d_input and wgrad partial tiles, in one grid or one after the other
    DgradBfArgs da{g, (const u16 *)dy, (const u16 *)ym, wpk, (u16 *)dx, relu, d,
                   make_fastdiv(g.OC * g.P)};
    WgradBfArgs wa{g, (const u16 *)x, dzg, part, wp};
    const int nx_dg = (g.B + d.G - 1) / d.G;
    const int n_dg = nx_dg * d.cgroups;
    const int n_wg = g.nxcd * ((wp.splits + g.nxcd - 1) / g.nxcd) * wp.ncol;
    if (p.fuse_main) {
        const int n_dg_pad = (n_dg + g.nxcd - 1) / g.nxcd * g.nxcd;
        hipLaunchKernelGGL(v->fn, dim3(n_dg_pad + n_wg), dim3(kWgNT), std::max(d.lds, wp.lds), s, da,
                           wa, n_dg, nx_dg, n_dg_pad);
    } else {
        hipLaunchKernelGGL(v->fn_d, dim3(nx_dg, d.cgroups), dim3(64 * d.NW), d.lds, s, da);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(v->fn_w, dim3(n_wg), dim3(2 * kWgNT), wp.lds, s, wa);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 3. fixed-order sum of the partial tiles
    return launch_wgrad_reduce<bf16_t>(part, dw, wp.splits, g.OC * g.K, s);
}

}  // namespace gc
