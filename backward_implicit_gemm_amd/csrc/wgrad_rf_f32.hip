// wgrad_rf_f32.hip -- weight gradient, fp32 storage, fp32 MFMA
// (v_mfma_f32_16x16x4_f32), both operands as single 16-byte LDS reads.
//
// dW[oc][k] = sum_r dz[r][oc] * x(r, k), r = (b, oh, ow), k = (ic, kh, kw):
// M = OC, N = IC*KH*KW, and a reduction over B*OH*OW split across
// workgroups.  The reduction runs over quads of 4 images: in a block of four
// MFMA steps, step j gives lane group q = lane/16 the element (position pair
// t = 4*blk + q, image j of that pair's quad), a pair being one (quad,
// output position) of the staging phase.  A lane's four steps therefore
// read the four images of one (quad, position), so both operands are staged
// in LDS images-innermost:
//   * dz (dy masked by y > 0 under ReLU) as [quad][oc][position][4 images],
//   * x as [quad][channel][pixel][4 images] (4x4 register transposes from
//     NCHW), read at pixel (oh*S + kh, ow*S + kw),
// and the A or B fragment of four steps is one ds_read_b128.
// A workgroup owns all OC rows and NBW 16-column blocks of k, and the quads
// of one split, which it walks in phases of QB quads through two LDS
// buffers.  Its 16 waves have two roles: waves 0..7 run the MFMAs (a 16-row
// oc block each, several waves per block when OC is small), waves 8..15 load,
// mask and transpose phase ph+1 into the other buffer while phase ph's MFMAs
// run, so the MFMA waves never wait on global memory.  Each workgroup writes
// its fp32 partial tile; wgrad_reduce.hip sums the partials in split order,
// so the result is deterministic.
#include "wgrad_rf_f32_dev.h"

namespace gc {
namespace {

struct WgradRfVariant {
    int NBWV;
    void (*fn[2][2])(WgradRfArgs);   // [relu: dz masked by y > 0][bias column]
};
#define WR_V(N)                                                                     \
    {N,                                                                             \
     {{wgrad_rf_f32<N, false, false>, wgrad_rf_f32<N, false, true>},                \
      {wgrad_rf_f32<N, true, false>, wgrad_rf_f32<N, true, true>}}}
const WgradRfVariant kWgradRfVariants[] = {WR_V(2), WR_V(3), WR_V(4), WR_V(6), WR_V(8)};
#undef WR_V

const WgradRfVariant *pick_wgrad_rf(int NBWV)
{
    for (const auto &v : kWgradRfVariants)
        if (v.NBWV == NBWV) return &v;
    return nullptr;
}

}  // namespace

// LDS bank cost of the B (x) fragment reads of a plan with x pitches WP, IS:
// for every 16-lane group of every read, the largest number of lanes whose
// 16-byte slots fall in the same 4-bank group, summed.
static int x_read_conflicts(const Geom &g, const WgradRfPlan &q, int WP, int IS)
{
    int cost = 0;
    for (int c = 0; c < q.chunks; ++c) {
        const int col0 = c * q.NBW * 16, c_lo = col0 / g.KK;
        for (int nb = 0; nb < q.NBW; ++nb)
            for (int s = 0; s < q.SPP; ++s)
                for (int qg = 0; qg < 4; ++qg) {
                    const int t = 4 * s + qg;
                    int xrow = 0;
                    if (t < q.QB * g.P) {
                        const int qb = t / g.P, pos = t % g.P;
                        xrow = qb * q.CCS * IS + (pos / g.OW) * g.S * WP + (pos % g.OW) * g.S;
                    }
                    int cnt[16] = {0}, worst = 0;
                    for (int l = 0; l < 16; ++l) {
                        const int col = col0 + nb * 16 + l;
                        if (col >= g.K) continue;
                        const int ic = col / g.KK, tap = col % g.KK;
                        const int slot = xrow + (ic - c_lo) * IS + (tap / g.KW) * WP + tap % g.KW;
                        worst = std::max(worst, ++cnt[slot & 15]);
                    }
                    cost += worst;
                }
    }
    return cost;
}

static bool plan_wgrad_rf_impl(const Geom &g, WgradRfPlan &p, int bias)
{
    const int MBLK = (g.OC + 15) / 16;
    if (MBLK > 8) return false;
    // the staging loads are 16-byte windows inside one image's dz and inside
    // the channels a chunk stages, and their 32-bit byte offsets reach at most
    // about twice the tensor size (images past the batch, unused units)
    if (g.OC * g.P < 4) return false;
    if ((2 * size_t(g.B) + 128) * g.IC * g.HW * 4 >= (size_t(1) << 32) ||
        (2 * size_t(g.B) + 128) * g.OC * g.P * 4 >= (size_t(1) << 32))
        return false;
    const int WN = MBLK == 1 ? 8 : MBLK == 2 ? 4 : MBLK <= 4 ? 2 : 1;
    const int NC = g.K + bias;              // computed columns
    const int NBT = (NC + 15) / 16;
    const int NQ = (g.B + 3) / 4;
    double best = 1e300;
    for (const auto &v : kWgradRfVariants) {
        WgradRfPlan q{};
        q.NBWV = v.NBWV; q.MBLK = MBLK; q.WN = WN; q.NBW = WN * v.NBWV;
        q.chunks = (NBT + q.NBW - 1) / q.NBW;
        q.NQ = NQ;
        q.bias = bias;
        q.NP = bias ? (g.K + 1 + 3) / 4 * 4 : g.K;
        q.CCS = 0;
        int min_span = 1 << 30;
        for (int c = 0; c < q.chunks; ++c) {
            const int lo = std::min(c * q.NBW * 16, g.K - 1);
            const int hi = std::min(g.K, (c + 1) * q.NBW * 16) - 1;
            q.CCS = std::max(q.CCS, hi / g.KK - lo / g.KK + 1);
            min_span = std::min(min_span, hi / g.KK - lo / g.KK + 1);
        }
        if (min_span * g.HW < 4) continue;
        q.XU = (q.CCS * g.HW + 3) / 4;
        q.DU = (g.OC * g.P + 3) / 4;
        q.OCP = g.OC;
        // the most quads per phase within four MFMA blocks and one staging
        // unit of each kind per thread
        q.QB = 0;
        for (int QB = 16; QB >= 1; --QB) {
            if ((QB * g.P + 3) / 4 > kSppMax || QB * q.XU > 512 || QB * q.DU > 512) continue;
            q.QB = QB;
            break;
        }
        if (!q.QB) continue;
        q.SPP = (q.QB * g.P + 3) / 4;
        // x pitches with the fewest LDS bank conflicts on the B reads, then
        // the smallest (independent of the batch size, so searched once per
        // layer shape and variant)
        static SearchMemo<std::pair<int, int>> memo;
        const int key[12] = {g.IC, g.H, g.W, g.OC, g.KH, g.KW, g.S, q.NBWV, q.QB, q.CCS, bias, 0};
        const std::pair<int, int> pitch = memo.get(key, [&] {
            int bc = 1 << 30, bw = g.W, bi = g.H * g.W;
            for (int WP = g.W; WP < g.W + 16; ++WP)
                for (int IS = g.H * WP; IS < g.H * WP + 16; ++IS) {
                    const int c = x_read_conflicts(g, q, WP, IS);
                    if (c < bc) { bc = c; bw = WP; bi = IS; }
                }
            return std::make_pair(bw, bi);
        });
        q.WP = pitch.first;
        q.IS = pitch.second;
        // x planes, dz, the zero slot (and with the bias column a slot of ones)
        q.bufsz = q.QB * q.CCS * q.IS + q.QB * g.P * q.OCP + 1 + bias;
        q.lds = size_t(2) * q.bufsz * 16;
        if (q.lds > 150 * 1024) continue;
        // one workgroup per CU: splits fill the CUs, in multiples of the
        // XCD count (one split per XCD)
        int splits = std::max(1, g.ncu / q.chunks);
        if (splits >= g.nxcd) splits -= splits % g.nxcd;
        splits = std::min({splits, NQ, 64});
        // a split's quads fill whole phases, so a phase never reaches into
        // the next split (only past the batch, where the loads return zeros)
        q.QPS = ((NQ + splits - 1) / splits + q.QB - 1) / q.QB * q.QB;
        q.splits = (NQ + q.QPS - 1) / q.QPS;
        const int nph = (q.QPS + q.QB - 1) / q.QB;
        // split z runs on XCD z % nxcd with all its chunks
        const double rounds = std::ceil(double((q.splits + g.nxcd - 1) / g.nxcd * q.chunks) /
                                        double(g.ncu / g.nxcd));
        // cycles per phase: two MFMA waves per SIMD at 32 cycles per MFMA,
        // but no less than the loader waves' fetch (a global load's latency)
        // and stash, plus ~200 for the barrier
        const double phase = std::max(2.0 * 4 * q.NBWV * q.SPP * 32, 3000.0) + 200.0;
        const double wg_cycles = nph * phase;
        const double part_bytes = 2.0 * q.splits * g.OC * double(q.NP) * 4;
        const double cost = rounds * wg_cycles + part_bytes / 5e12 * 2.4e9;
        q.ws_bytes = size_t(q.splits) * g.OC * q.NP * sizeof(float);
        if (cost < best) {
            best = cost;
            p = q;
        }
    }
    return best < 1e300;
}

bool plan_wgrad_rf_f32(const Geom &g, WgradRfPlan &p) { return plan_wgrad_rf_impl(g, p, 0); }
bool plan_wgrad_rf_f32_bias(const Geom &g, WgradRfPlan &p) { return plan_wgrad_rf_impl(g, p, 1); }

hipError_t launch_wgrad_rf_f32(const Geom &g, const WgradRfPlan &p, const void *x, const void *dy,
                               const void *ym, void *dw, void *db, void *ws, int relu, hipStream_t s)
{
    if (p.bias && !db) return hipErrorInvalidValue;
    const WgradRfVariant *v = pick_wgrad_rf(p.NBWV);
    if (!v || p.QB * p.XU > 512 || p.QB * p.DU > 512 || p.SPP > kSppMax)
        return hipErrorInvalidValue;
    if (reinterpret_cast<uintptr_t>(ws) % 16) return hipErrorInvalidValue;
    WgradRfArgs a{g, (const float *)x, (const float *)dy, (const float *)ym, (float *)ws, relu, p};
    void (*fn)(WgradRfArgs) = v->fn[relu ? 1 : 0][p.bias ? 1 : 0];
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(fn));
    if (e != hipSuccess) return e;
    const int grid = g.nxcd * ((p.splits + g.nxcd - 1) / g.nxcd) * p.chunks;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(1024), p.lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.bias) return launch_wgrad_reduce_bias<float>((const float *)ws, dw, db, p.splits, g.OC, g.K, p.NP, s);
    return launch_wgrad_reduce<float>((const float *)ws, dw, p.splits, g.OC * g.K, s);
}

}  // namespace gc
