// dgrad_ig_bf16.hip -- d_input, bf16 storage, bf16 MFMA with fp32 accumulation,
// image-group tiling, gather form (no atomics, each dx element written once).
//
// A workgroup owns G whole images (G a multiple of 4).  Their masked output
// gradient dz = dy * (y > 0) (just dy without a ReLU) is staged once in LDS as
// rows m = p*G + img (the image index innermost) by columns oc, and every wave
// then holds the A fragments of all its rows for the whole reduction over oc
// in registers.  The input channels are walked in chunks of CC; for each
// chunk the column gradient
//     dcol[m][(icl,kh,kw)] = sum_oc dz[m][oc] * w[oc][c0+icl][kh][kw]
// is formed on v_mfma_f32_16x16x32_bf16 with the waves splitting its 16-column
// blocks.  The weights are pre-packed (a small kernel before the main one)
// into the exact B-fragment order -- [chunk][column block][32-oc step][lane]
// x 8 oc -- so a wave's B operand for one step is one contiguous 1 KB load,
// requested one chunk ahead of its use.  The fp32 dcol tile goes to LDS, column
// by column, and the chunk's input gradient is gathered from it:
//     dx[b][ic][ih][iw] = sum over the taps with oh*S+kh = ih, ow*S+kw = iw
//                         of dcol[(oh,ow,b)][(ic,kh,kw)]
// Because the image index is innermost in m, one 16-byte LDS read returns a
// tap for four images at once.  The sum is in fp32 in a fixed tap order and
// rounded to bf16 once into an LDS tile of the chunk's dx, which leaves in
// 16-byte stores after the next barrier.  dcol and the dx tile are
// double-buffered, so one barrier per chunk separates every LDS producer from
// its consumers.  Index arithmetic is
// 32-bit (the C ABI caps every tensor below 2^31 elements).
#include "dgrad_ig_bf16_dev.h"

namespace gc {
namespace {

struct DgradBfVariant {
    int NW, MB, KS, TAPS, NBW, GP;
    void (*fn)(DgradBfArgs);
};

// GP (gather passes per chunk) is 2 throughout: the planner keeps every
// chunk's planes within two passes of the gather threads.
#define DB_V(MB, KS, TAPS, NBW) {8, MB, KS, TAPS, NBW, 2, dgrad_ig_bf16<8, MB, KS, TAPS, NBW, 2>}
#define DB_NBW(MB, KS, TAPS) DB_V(MB, KS, TAPS, 1), DB_V(MB, KS, TAPS, 2)
#define DB_TAPS(MB, KS) DB_NBW(MB, KS, 2), DB_NBW(MB, KS, 4), DB_NBW(MB, KS, 9)
#define DB_KS(MB) DB_TAPS(MB, 1), DB_TAPS(MB, 2), DB_TAPS(MB, 4)
const DgradBfVariant kDgradBfVariants[] = {DB_KS(1), DB_KS(2), DB_KS(3), DB_KS(4)};
#undef DB_KS
#undef DB_TAPS
#undef DB_NBW
#undef DB_V

const DgradBfVariant *pick_dgrad_bf(int NW, int MB, int KS, int TAPS, int NBW, int GP)
{
    for (const auto &v : kDgradBfVariants)
        if (v.NW == NW && v.MB == MB && v.KS == KS && v.TAPS == TAPS && v.NBW == NBW && v.GP == GP)
            return &v;
    return nullptr;
}

// Most taps any input pixel receives.
int max_taps(const Geom &g)
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

// Picks the image-group size G (a multiple of 4), the channel chunk CC and the
// split of the chunks over workgroups from a cycle estimate of the MFMA work
// per wave, the gather's LDS reads and a fixed cost per chunk barrier.
bool plan_dgrad_ig_bf16(const Geom &g, DgradBfPlan &p)
{
    constexpr int NW = 8, NT = 64 * NW;
    if (g.HW > NT || g.P > 16) return false;
    int KS = (g.OC + 31) / 32;
    if (KS > 4) return false;
    if (KS == 3) KS = 4;
    const int mt = max_taps(g);
    const int TAPS = mt <= 2 ? 2 : mt <= 4 ? 4 : mt <= 9 ? 9 : 0;
    if (!TAPS) return false;
    const int rpi = NT / g.HW;
    double best = 1e30;
    bool found = false;
    for (int G = 4; G <= 64; G += 4) {
        const int MB = (G * g.P + 15) / 16;
        if (MB > 4) break;
        if (G > 4 && G - 4 >= g.B) break;   // no larger group than the batch needs
        const int OCP = 32 * KS + 8;
        // column pitch: MB*16 computed rows, G zero rows, and RP/4 odd so the
        // 16-byte column writes of 16 lanes hit distinct bank groups
        const int RP = MB * 16 + G + (((G / 4) & 1) ? 0 : 4);
        const size_t dz_bytes = size_t(MB) * 16 * OCP * 2;
        const int ngroups = (g.B + G - 1) / G;
        for (int CC = 1; CC <= g.IC; ++CC) {
            const int NBC = (CC * g.KK + 15) / 16;
            const int NBW = (NBC + NW - 1) / NW;
            if (NBW > 2) break;
            const int GP = 2;
            if (CC * (G / 4) > GP * rpi) break;
            const int ORUN = (CC * g.HW + 7) & ~7;
            const size_t lds = dz_bytes + 2 * size_t(NBC) * 16 * RP * 4 + 2 * size_t(G) * ORUN * 2;
            if (lds > 160 * 1024) break;
            const int nchunks = (g.IC + CC - 1) / CC;
            const int occ = lds <= 80 * 1024 ? 2 : 1;
            int cgroups = 1;
            while (ngroups * cgroups < g.ncu * occ && cgroups < nchunks) ++cgroups;
            const int cpg = (nchunks + cgroups - 1) / cgroups;
            cgroups = (nchunks + cpg - 1) / cpg;
            // cycles per chunk on one CU
            const double mfma = double((NBC + NW - 1) / NW) * MB * KS * 16 * (NW / 4);
            const double passes = double((CC * (G / 4) + rpi - 1) / rpi);
            const double gather = passes * NW * (mt * 8.0 + 16.0);
            const double chunk = mfma + gather + 400.0;
            const double per_wg = cpg * chunk + 2500.0;
            const double waves_of_wgs = std::ceil(double(ngroups) * cgroups / (double(g.ncu) * occ));
            const double t = waves_of_wgs * per_wg * (occ == 2 ? 1.4 : 1.0);
            if (t < best - 1e-9) {
                if (!pick_dgrad_bf(NW, MB, KS, TAPS, NBW, GP)) continue;
                best = t;
                p.NW = NW; p.G = G; p.MB = MB; p.KS = KS; p.TAPS = TAPS; p.NBW = NBW; p.GP = GP;
                p.CC = CC; p.NBC = NBC; p.nchunks = nchunks; p.cgroups = cgroups; p.cpg = cpg;
                p.RP = RP; p.OCP = OCP; p.dz_bytes = int(dz_bytes); p.ORUN = ORUN;
                p.lds = lds;
                p.ws_bytes = size_t(nchunks) * NBC * KS * 64 * 16;
                found = true;
            }
        }
    }
    return found;
}

hipError_t launch_dgrad_ig_bf16(const Geom &g, const DgradBfPlan &p, const void *dy, const void *w,
                                const void *ym, void *dx, void *ws, int relu, hipStream_t s)
{
    const DgradBfVariant *v = pick_dgrad_bf(p.NW, p.MB, p.KS, p.TAPS, p.NBW, p.GP);
    if (!v || g.HW > 64 * p.NW || p.G % 4 || p.G * g.P > 16 * p.MB || p.NBC > p.NW * p.NBW ||
        p.RP < 16 * p.MB + p.G || p.CC * (p.G / 4) > p.GP * ((64 * p.NW) / g.HW))
        return hipErrorInvalidValue;
    const int total = p.nchunks * p.NBC * p.KS * 64;
    if (size_t(total) * 16 > p.ws_bytes) return hipErrorInvalidValue;
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pack_w_dgrad_bf16, dim3(std::min((total + 255) / 256, 2048)), dim3(256), 0, s,
                       (const u16 *)w, (uint4 *)ws, g, p.CC, make_fastdiv(p.NBC), make_fastdiv(p.KS),
                       total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    DgradBfArgs a{g, (const u16 *)dy, (const u16 *)ym, (const uint4 *)ws, (u16 *)dx, relu, p,
                  make_fastdiv(g.OC * g.P)};
    dim3 grid((g.B + p.G - 1) / p.G, p.cgroups);
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
