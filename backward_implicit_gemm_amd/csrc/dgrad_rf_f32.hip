// dgrad_rf_f32.hip -- d_input, fp32 storage, fp32 MFMA (v_mfma_f32_16x16x4_f32),
// image-group tiling, gather form (no atomics, each dx element written once).
//
// Same structure as the bf16 d_input kernel: a workgroup owns G whole images
// (G a multiple of 4) and stages their masked output gradient dz once in LDS
// as rows m = p*G + img by columns oc.  Input channels are walked in chunks of
// CC; for each chunk the column gradient
//     dcol[m][(icl,kh,kw)] = sum_oc dz[m][oc] * w[oc][c0+icl][kh][kw]
// is formed by eight MFMA waves (two per SIMD), one 16-column block each,
// while eight gather waves gather the previous chunk (see the kernel).  The
// reduction over oc runs in blocks of 16 channels, MFMA step j giving lane
// group q the channel 16*s + 4*q + j, so a lane's A values for four steps are
// one 16-byte LDS read of its dz row; its B values are four floats of w read
// in place (16 lanes read 16 consecutive floats of one weight row), a few
// channel blocks ahead of their MFMAs.  dcol goes to LDS column by column and
// the chunk's input gradient is gathered from it, four images per 16-byte read:
//     dx[b][ic][ih][iw] = sum over the taps with oh*S+kh = ih, ow*S+kw = iw
//                         of dcol[(oh,ow,b)][(ic,kh,kw)]
// in fp32 in a fixed tap order and stored straight to dx (64 consecutive
// pixels per store instruction).  dcol is double-buffered, so one barrier per
// chunk separates its writers from its readers.
// Only taps that land on an output position are multiplied (algorithmic MACs).
#include "dgrad_rf_f32_dev.h"

namespace gc {
namespace {

struct DgradRfVariant {
    int NW, MB, KS4, TAPS, NBW;
    bool exact;          // OC == 16*KS4
    void (*fn)(DgradRfArgs);
};

#define DR_V(MB, KS4, TAPS, EX) {16, MB, KS4, TAPS, 1, EX, dgrad_rf_f32<MB, KS4, TAPS, 1, EX>}
#define DR_TAPS(MB, KS4, EX) DR_V(MB, KS4, 2, EX), DR_V(MB, KS4, 4, EX), DR_V(MB, KS4, 9, EX)
#define DR_MB(KS4, EX) DR_TAPS(1, KS4, EX), DR_TAPS(2, KS4, EX), DR_TAPS(3, KS4, EX)
const DgradRfVariant kDgradRfVariants[] = {
    DR_MB(8, true), DR_MB(4, true), DR_MB(2, true), DR_MB(1, true),        // OC 128, 64, 32, 16
    DR_MB(8, false), DR_MB(4, false), DR_MB(2, false), DR_MB(1, false),    // OC below those
};
#undef DR_MB
#undef DR_TAPS
#undef DR_V

const DgradRfVariant *pick_dgrad_rf(int NW, int MB, int KS4, int TAPS, int NBW, bool exact)
{
    for (const auto &v : kDgradRfVariants)
        if (v.NW == NW && v.MB == MB && v.KS4 == KS4 && v.TAPS == TAPS && v.NBW == NBW && v.exact == exact)
            return &v;
    return nullptr;
}

// Most taps any input pixel receives.
int max_taps_rf(const Geom &g)
{
    int best = 0;
    for (int ih = 0; ih < g.H; ++ih)
        for (int iw = 0; iw < g.W; ++iw) {
            int n = 0;
            for (int oh = 0; oh < g.OH; ++oh) {
                const int kh = ih - oh * g.S;
                if (kh < 0 || kh >= g.KH) continue;
                for (int ow = 0; ow < g.OW; ++ow) {
                    const int kw = iw - ow * g.S;
                    if (kw >= 0 && kw < g.KW) ++n;
                }
            }
            best = std::max(best, n);
        }
    return best;
}

}  // namespace

// Eight MFMA waves take one column block each per chunk (NBC <= 8); the
// chunk time is the longer of their MFMA work (two waves per SIMD) and the
// gather waves' work.  MB is capped at 3.
bool plan_dgrad_rf_f32(const Geom &g, DgradBfPlan &p)
{
    constexpr int NW = 16, NGT = 512;
    if (g.HW > NGT || g.P > 16) return false;
    // dx and w byte offsets are 32-bit offsets inside their tensors
    if (size_t(g.B) * g.IC * g.HW * 4 >= (size_t(1) << 31) || size_t(g.OC) * g.K * 4 >= (size_t(1) << 31))
        return false;
    const int ks4 = (g.OC + 15) / 16;
    const int KS4 = ks4 <= 1 ? 1 : ks4 <= 2 ? 2 : ks4 <= 4 ? 4 : ks4 <= 8 ? 8 : 0;
    if (!KS4) return false;
    const int mt = max_taps_rf(g);
    const int TAPS = mt <= 2 ? 2 : mt <= 4 ? 4 : mt <= 9 ? 9 : 0;
    if (!TAPS) return false;
    const int rpi = NGT / g.HW;
    double best = 1e30;
    bool found = false;
    for (int G = 4; G <= 64; G += 4) {
        const int MB = (G * g.P + 15) / 16;
        if (MB > 3) break;
        if (G > 4 && G - 4 >= g.B) break;
        const int OCP = 16 * KS4 + 4;     // A-fragment reads: bank 4*row + lane/16, no conflicts
        const int RP = MB * 16 + G + (((G / 4) & 1) ? 0 : 4);
        const size_t dz_bytes = size_t(MB) * 16 * OCP * 4;
        const int ngroups = (g.B + G - 1) / G;
        for (int CC = 1; CC <= g.IC; ++CC) {
            const int NBC = (CC * g.KK + 15) / 16;
            if (NBC > 8) break;
            if ((CC * (G / 4) + rpi - 1) / rpi > 4) break;   // planes per gather thread
            const int NBW = 1;
            const size_t lds = dz_bytes + 2 * size_t(NBC) * 16 * RP * 4;
            if (lds > 160 * 1024) break;
            const int nchunks = (g.IC + CC - 1) / CC;
            int cgroups = 1;
            while (ngroups * cgroups < g.ncu && cgroups < nchunks) ++cgroups;
            const int cpg = (nchunks + cgroups - 1) / cgroups;
            cgroups = (nchunks + cpg - 1) / cpg;
            const double mfma = 2.0 * MB * 4 * KS4 * 32;
            const double passes = double((CC * (G / 4) + rpi - 1) / rpi);
            const double gather = passes * 4 * (mt * 16.0 + 40.0) + 600.0;
            const double chunk = std::max(mfma, gather) + 300.0;
            const double per_wg = cpg * chunk + 2500.0;
            const double t = std::ceil(double(ngroups) * cgroups / double(g.ncu)) * per_wg;
            if (t < best - 1e-9) {
                if (!pick_dgrad_rf(NW, MB, KS4, TAPS, NBW, g.OC == 16 * KS4)) continue;
                best = t;
                p.NW = NW; p.G = G; p.MB = MB; p.KS = KS4; p.TAPS = TAPS; p.NBW = NBW; p.GP = 0;
                p.CC = CC; p.NBC = NBC; p.nchunks = nchunks; p.cgroups = cgroups; p.cpg = cpg;
                p.RP = RP; p.OCP = OCP; p.dz_bytes = int(dz_bytes); p.ORUN = 0;
                p.lds = lds;
                p.ws_bytes = 0;
                found = true;
            }
        }
    }
    return found;
}

hipError_t launch_dgrad_rf_f32(const Geom &g, const DgradBfPlan &p, const void *dy, const void *w,
                               const void *ym, void *dx, int relu, hipStream_t s)
{
    const DgradRfVariant *v = pick_dgrad_rf(p.NW, p.MB, p.KS, p.TAPS, p.NBW, g.OC == 16 * p.KS);
    if (!v || p.NW != 16 || g.HW > 512 || p.G % 4 || p.G * g.P > 16 * p.MB || p.NBC > 8 * p.NBW ||
        p.RP < 16 * p.MB + p.G)
        return hipErrorInvalidValue;
    // at most four planes per gather thread and chunk; dx and w byte offsets
    // are 32-bit offsets inside their tensors
    const int rpi = 512 / g.HW;
    if ((p.CC * (p.G / 4) + rpi - 1) / rpi > 4 || size_t(g.OC) * g.K * 4 >= (size_t(1) << 31) ||
        size_t(g.B) * g.IC * g.HW * 4 >= (size_t(1) << 31))
        return hipErrorInvalidValue;
    DgradRfArgs a{g, (const float *)dy, (const float *)ym, (const float *)w, (float *)dx, relu, p,
                  make_fastdiv(g.OC * g.P)};
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    dim3 grid((g.B + p.G - 1) / p.G, p.cgroups);
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
