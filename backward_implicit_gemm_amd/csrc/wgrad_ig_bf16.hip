// wgrad_ig_bf16.hip -- weight gradient, bf16 storage, bf16 MFMA with fp32
// accumulation, split-K over groups of 8 images.
//
//     dw[oc][n] = sum over (b, p) of dz[b][oc][p] * x[b][ic][oh*S+kh][ow*S+kw],
//     n = (ic, kh, kw), p = (oh, ow), dz = dy * (y > 0) (dy without a ReLU).
//
// The reduction index is ordered (8-image group, position p, image within
// the group): one v_mfma_f32_16x16x32_bf16 step covers 4 positions x 8
// images, and each lane's 8 consecutive reduction elements are the 8 images
// of one (oc, p) or one (n, p), so both operands are single 16-byte LDS
// reads once the data is staged image-innermost:
//   * a pre-pass writes dz as [group][p][oc][8 images] (positions padded to a
//     multiple of 4 and channels to 128 with zeros), so a workgroup's dz stage
//     for one group is a contiguous 16-byte copy;
//   * x is staged per group as [channel][pixel][8 images]: a thread loads 8
//     pixels of one channel for each of the 8 images and transposes the 8x8
//     block in registers.
// A workgroup owns 128 output channels x 64*JW columns (8 waves of 64 x
// 16*JW) and a contiguous range of image groups, pipelined three deep: one group's
// operands in LDS feeding the MFMAs, the next group's in registers, and the
// loads of the one after in flight.  It writes its fp32 partial tile, and a
// fixed-order sum over the ranges finishes dw (deterministic, no atomics).
#include "wgrad_ig_bf16_dev.h"

namespace gc {
namespace {

// The role-split kernel (16 waves) runs the standalone call.
struct WgradBfVariant {
    int NSTEP, JW;
    void (*fn[2])(WgradBfArgs);     // [bias column]
};
#define WB_V(NSTEP, JW) {NSTEP, JW, {wgrad_ws_bf16<NSTEP, JW, false>, wgrad_ws_bf16<NSTEP, JW, true>}}
const WgradBfVariant kWgradBfVariants[] = {
    WB_V(1, 2), WB_V(1, 4), WB_V(2, 2), WB_V(2, 4),
    WB_V(3, 2), WB_V(3, 4), WB_V(4, 2), WB_V(4, 4),
};
#undef WB_V

const WgradBfVariant *pick_wgrad_bf(int nstep, int jw)
{
    for (const auto &v : kWgradBfVariants)
        if (v.NSTEP == nstep && v.JW == jw) return &v;
    return nullptr;
}

}  // namespace

// The plan for column tiles of 64*JW columns (JW 16-column blocks per MFMA
// wave), image groups of 8 split over `splits` workgroup rows.  The number
// of splits trades MFMA parallelism (at least ~one workgroup per CU) against
// the fp32 partial traffic (splits x OC x K x 4 bytes, written and read
// back once).
bool plan_wgrad_bf16_tiles(const Geom &g, int JW, WgradBfPlan &p, int bias)
{
    if (g.OC > 128 || g.P > 16 || g.HW < 8) return false;
    const int PP = (g.P + 3) / 4 * 4;
    const int NSTEP = PP / 4;
    if (!pick_wgrad_bf(NSTEP, JW)) return false;
    const int N = g.K, TW = 64 * JW;
    const int ncol = (N + bias + TW - 1) / TW;     // the bias is column N
    // widest channel span of any tile
    int CCW = 0;
    for (int t = 0; t < ncol; ++t) {
        const int lo = std::min(t * TW, N - 1) / g.KK;
        const int hi = std::min(g.IC - 1, (std::min(N, t * TW + TW) - 1) / g.KK);
        CCW = std::max(CCW, hi - lo + 1);
    }
    const int nblk = (g.HW + 7) / 8;
    if (2 * CCW * nblk > kWgNT) return false;
    const int HWP = nblk * 9;        // 8-pixel blocks of 9 LDS slots (see xslot)
    // two stages of x (plus the bias column's unit of ones) and dz
    const size_t lds = 2 * (size_t(CCW) * HWP + (bias ? 1 : 0) + size_t(PP) * 128) * 16;
    if (lds > 160 * 1024) return false;
    const int ngroups = (g.B + 7) / 8;
    // splits: enough workgroups to cover the CUs, in multiples of the XCD
    // count so the XCDs get equal shares, few enough that the partial
    // traffic stays small against the operand traffic
    int splits = std::max(1, std::min(ngroups, (g.ncu + ncol - 1) / ncol));
    if (splits > g.nxcd) splits = splits / g.nxcd * g.nxcd;
    const int NP = bias ? (N + 1 + 3) / 4 * 4 : N;
    const double part_bytes = double(g.OC) * NP * 4;
    const double in_bytes = double(g.B) * g.IC * g.HW * 2;
    const double budget = std::max(0.75 * in_bytes, 12.0 * 1024 * 1024);
    while (splits > g.nxcd && splits * part_bytes > budget) splits -= g.nxcd;
    while (splits > 1 && splits <= g.nxcd && splits * part_bytes > budget) --splits;
    const int gps = (ngroups + splits - 1) / splits;
    splits = (ngroups + gps - 1) / gps;
    p.NSTEP = NSTEP; p.JW = JW; p.bias = bias; p.NP = NP;
    p.PP = PP; p.CCW = CCW; p.nblk = nblk; p.HWP = HWP;
    p.ncol = ncol; p.ngroups = ngroups; p.gps = gps; p.splits = splits;
    p.lds = lds;
    p.dz_bytes = (size_t(ngroups) * PP * 128 * 16 + 255) / 256 * 256;
    p.ws_bytes = p.dz_bytes + size_t(splits) * g.OC * NP * 4;
    return true;
}

// Tiles of 256 columns (JW = 4) stage dz for half as many tiles per 8-image
// group, so each workgroup moves fewer bytes from L2 per MFMA; but with half
// the tiles the chip fills only when the batch allows about twice the
// splits, and a workgroup with no more splits to share does twice the work
// per group.  They are taken when their grid covers the CUs (the chain's
// B=16384: conv1 wgrad 184 -> 144 us, conv2 67 -> 51 us); below that (B=1024:
// 96 workgroups, 26.8 -> 30.2 us) the 128-column tiles run.
static bool plan_wgrad_bf16(const Geom &g, WgradBfPlan &p, int bias)
{
    WgradBfPlan q{};
    if (plan_wgrad_bf16_tiles(g, 4, q, bias) && 10 * q.ncol * q.splits >= 9 * g.ncu) {
        p = q;
        return true;
    }
    return plan_wgrad_bf16_tiles(g, 2, p, bias);
}

bool plan_wgrad_ig_bf16(const Geom &g, WgradBfPlan &p) { return plan_wgrad_bf16(g, p, 0); }
bool plan_wgrad_ig_bf16_bias(const Geom &g, WgradBfPlan &p) { return plan_wgrad_bf16(g, p, 1); }

hipError_t launch_wgrad_ig_bf16(const Geom &g, const WgradBfPlan &p, const void *x, const void *dy,
                                const void *ym, void *dw, void *db, void *ws, int relu, hipStream_t s)
{
    if (p.bias && !db) return hipErrorInvalidValue;
    hipError_t e;
    const WgradBfVariant *v = pick_wgrad_bf(p.NSTEP, p.JW);
    if (!v || 2 * p.CCW * p.nblk > kWgNT || p.PP * 128 != p.NSTEP * kWgNT || g.OC > 128 || g.HW < 8)
        return hipErrorInvalidValue;
    uint4 *dzg = static_cast<uint4 *>(ws);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + p.dz_bytes);
    const size_t dz_lds = dz_groups_lds(g);
    if (kDzOC * g.P > kDzChunks * kDzNT) return hipErrorInvalidValue;
    e = allow_max_lds(reinterpret_cast<const void *>(&dz_groups_bf16));
    if (e != hipSuccess) return e;
    void (*fn)(WgradBfArgs) = v->fn[p.bias ? 1 : 0];
    e = allow_max_lds(reinterpret_cast<const void *>(fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dz_groups_bf16, dim3(p.ngroups * kDzSlices), dim3(kDzNT), dz_lds, s,
                       (const u16 *)dy, (const u16 *)ym, dzg, g, relu, p.PP);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    WgradBfArgs a{g, (const u16 *)x, dzg, part, p};
    const int slots = (p.splits + g.nxcd - 1) / g.nxcd * p.ncol;    // per XCD
    hipLaunchKernelGGL(fn, dim3(g.nxcd * slots), dim3(2 * kWgNT), p.lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.bias) return launch_wgrad_reduce_bias<bf16_t>(part, dw, db, p.splits, g.OC, g.K, p.NP, s);
    return launch_wgrad_reduce<bf16_t>(part, dw, p.splits, g.OC * g.K, s);
}

}  // namespace gc
