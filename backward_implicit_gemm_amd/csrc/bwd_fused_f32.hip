// bwd_fused_f32.hip -- the fp32 backward (d_input and wgrad) in two launches
// instead of three.
//
// The separate calls launch the d_input kernel, the wgrad partial-tile kernel
// and the fixed-order reduction.  Here the d_input workgroups and the wgrad
// workgroups share one grid: the two sets are independent (both read dy and
// the mask, d_input also w, wgrad also x), so wgrad workgroups start on the
// CUs that d_input workgroups leave, without the drain and launch gap between
// two kernels.  Both kernels run 16 waves per workgroup, one workgroup per
// CU, so one grid costs neither of them occupancy.  The reduction stays a
// launch of its own (summing in split order needs every partial tile).
// Both bodies are the ones the separate calls run, so dx and dw are
// bit-identical to gc_conv_bwd_data + gc_conv_bwd_weight.
#include "dgrad_rf_f32_dev.h"
#include "wgrad_rf_f32_dev.h"

namespace gc {
namespace {

// d_input workgroups first (n_dg of them, an (image group, chunk group) grid
// of nx_dg columns, padded to a multiple of the XCD count), then the wgrad
// workgroups; the padding keeps each wgrad workgroup on the XCD its own
// decode expects (workgroup ids go round-robin over the XCDs).
template <int MB, int KS4, int TAPS, bool EXACT, int NBWV, bool RELU>
__global__ void __launch_bounds__(1024) bwd_fused_f32(DgradRfArgs da, WgradRfArgs wa, int n_dg,
                                                      int nx_dg, int n_dg_pad)
{
    const int bid = blockIdx.x;
    if (bid < n_dg)
        dgrad_rf_f32_body<MB, KS4, TAPS, 1, EXACT>(da, bid % nx_dg, bid / nx_dg);
    else if (bid >= n_dg_pad)
        wgrad_rf_f32_body<NBWV, RELU, false>(wa, bid - n_dg_pad);
}

struct FusedF32Variant {
    int MB, KS4, TAPS, NBWV;
    bool exact;
    void (*fn[2])(DgradRfArgs, WgradRfArgs, int, int, int);   // [relu]
};
// The (d_input, wgrad) kernel pairs the planners choose for the policy
// network's layers; other shapes use the separate calls.
#define FF(MB, KS4, TAPS, EX, NBWV)                                                      \
    {MB, KS4, TAPS, NBWV, EX,                                                            \
     {bwd_fused_f32<MB, KS4, TAPS, EX, NBWV, false>, bwd_fused_f32<MB, KS4, TAPS, EX, NBWV, true>}}
const FusedF32Variant kFusedF32Variants[] = {
    FF(3, 8, 4, true, 6), FF(3, 8, 4, true, 3),                         // 59 -> 128, 11x15, 5x5, stride 3
    FF(1, 8, 2, true, 3), FF(2, 8, 2, true, 3), FF(3, 8, 2, true, 3),   // 128 -> 128, 3x4, 3x3
};
#undef FF

const FusedF32Variant *pick_fused_f32(const Geom &g, const DgradBfPlan &d, const WgradRfPlan &w)
{
    if (d.NW != 16 || d.NBW != 1) return nullptr;
    for (const auto &v : kFusedF32Variants)
        if (v.MB == d.MB && v.KS4 == d.KS && v.TAPS == d.TAPS && v.exact == (g.OC == 16 * d.KS) &&
            v.NBWV == w.NBWV)
            return &v;
    return nullptr;
}

}  // namespace

bool plan_bwd_fused_f32(const Geom &g, BwdFusedF32Plan &p)
{
    BwdFusedF32Plan q{};
    if (!plan_dgrad_rf_f32(g, q.d) || !plan_wgrad_rf_f32(g, q.w)) return false;
    if (q.w.bias || q.w.MBLK * q.w.WN > 8 || !pick_fused_f32(g, q.d, q.w)) return false;
    q.ws_bytes = q.w.ws_bytes;
    p = q;
    return true;
}

hipError_t launch_bwd_fused_f32(const Geom &g, const BwdFusedF32Plan &p, const void *x,
                                const void *w, const void *dy, const void *ym, void *dx, void *dw,
                                void *ws, int relu, hipStream_t s)
{
    const DgradBfPlan &d = p.d;
    const WgradRfPlan &wp = p.w;
    const FusedF32Variant *v = pick_fused_f32(g, d, wp);
    if (!v || wp.bias) return hipErrorInvalidValue;
    // the preconditions of the two kernels, as their own launches check them
    const int rpi = 512 / g.HW;
    if (g.HW > 512 || d.G % 4 || d.G * g.P > 16 * d.MB || d.NBC > 8 || d.RP < 16 * d.MB + d.G ||
        (d.CC * (d.G / 4) + rpi - 1) / rpi > 4 || size_t(g.OC) * g.K * 4 >= (size_t(1) << 31) ||
        size_t(g.B) * g.IC * g.HW * 4 >= (size_t(1) << 31))
        return hipErrorInvalidValue;
    if (wp.QB * wp.XU > 512 || wp.QB * wp.DU > 512 || wp.SPP > kSppMax || wp.MBLK * wp.WN > 8)
        return hipErrorInvalidValue;
    if (reinterpret_cast<uintptr_t>(ws) % 16) return hipErrorInvalidValue;

    auto fn = v->fn[relu ? 1 : 0];
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(fn));
    if (e != hipSuccess) return e;
    float *part = static_cast<float *>(ws);
    DgradRfArgs da{g, (const float *)dy, (const float *)ym, (const float *)w, (float *)dx, relu, d,
                   make_fastdiv(g.OC * g.P)};
    WgradRfArgs wa{g, (const float *)x, (const float *)dy, (const float *)ym, part, relu, wp};
    const int nx_dg = (g.B + d.G - 1) / d.G;
    const int n_dg = nx_dg * d.cgroups;
    const int n_dg_pad = (n_dg + g.nxcd - 1) / g.nxcd * g.nxcd;
    const int n_wg = g.nxcd * ((wp.splits + g.nxcd - 1) / g.nxcd) * wp.chunks;
    hipLaunchKernelGGL(fn, dim3(n_dg_pad + n_wg), dim3(1024), std::max(d.lds, wp.lds), s, da, wa,
                       n_dg, nx_dg, n_dg_pad);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_wgrad_reduce<float>(part, dw, wp.splits, g.OC * g.K, s);
}

}  // namespace gc
