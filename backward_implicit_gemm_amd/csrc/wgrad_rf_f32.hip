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
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

constexpr int kSppMax = 4;     // 4-step MFMA blocks per phase, at most

struct WgradRfArgs {
    Geom g;
    const float *x, *dy, *ym;
    float *part;
    int relu;
    WgradRfPlan p;
};

__device__ __forceinline__ float comp(const float4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}


template <int NBWV, bool RELU, bool BIAS>
__global__ void __launch_bounds__(1024) wgrad_rf_f32(WgradRfArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float4 lds4w[];
    const Geom &g = a.g;
    const WgradRfPlan &p = a.p;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // waves 0..7 run the MFMAs, waves 8..15 stage the operands
    const bool loader = wave >= 8;
    const int ltid = tid - 512;                     // loader thread index

    // Workgroups are dealt to the XCDs round-robin by id; all column chunks
    // of one split share an XCD, whose L2 then serves that split's dz to
    // every chunk.
    const int nx = a.g.nxcd;
    const int xcd = int(blockIdx.x) % nx, slot = int(blockIdx.x) / nx;
    const int split = (slot / p.chunks) * nx + xcd;
    if (split >= p.splits) return;
    const int chunk = slot % p.chunks;
    const int qs = split * p.QPS;
    const int qe = min(p.NQ, qs + p.QPS);
    const int nph = qe > qs ? (qe - qs + p.QB - 1) / p.QB : 0;
    const int col0 = chunk * p.NBW * 16;
    // (a chunk holding only the bias column stages channel IC-1, unused)
    const int c_lo = int(fdiv(uint32_t(min(col0, g.K - 1)), g.fd_KK));
    const int c_hi = min(g.IC - 1, int(fdiv(uint32_t(min(g.K, col0 + p.NBW * 16) - 1), g.fd_KK)));
    const int QX = p.CCS * p.IS, QD = g.P * p.OCP;  // LDS slots per quad: x, dz
    const int xsz = p.QB * QX;                      // x slots of a buffer
    const int zslot = xsz + p.QB * QD;              // the buffer's zero slot

    // Staging units, one of each kind per thread at most.  The chunk's
    // channels of one image are contiguous in NCHW, and so is one image's dz,
    // so a unit is 4 consecutive elements of one of them (a channel or row
    // boundary may fall inside) for the 4 images of a quad:
    //   x unit  (quad, block of the image's staged channels [c_lo, c_hi])
    //   dz unit (quad, block of the image's OC*P dz elements)
    // The last block of a range is moved back to end with it (it rewrites
    // some of its neighbour's slots with the same values), so every load is
    // 16 bytes inside one image.  Images past the batch read past the end of
    // their tensor and load zeros.
    const int xlen = (c_hi - c_lo + 1) * g.HW, dlen = g.OC * g.P;
    const int lu = loader ? ltid : 0;
    const int x_qb = lu / p.XU, x_f0 = min(4 * (lu % p.XU), xlen - 4);
    const bool x_act = loader && ltid < p.QB * p.XU && 4 * (lu % p.XU) < xlen;
    const int d_qb = lu / p.DU, d_f0 = min(4 * (lu % p.DU), dlen - 4);
    const bool d_act = loader && ltid < p.QB * p.DU;
    int xs[4], ds[4];     // LDS slots of the unit's elements
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t cs, pix, ih, iw, oc, pos;
        fdivmod(uint32_t(x_f0 + e), g.fd_HW, cs, pix);
        fdivmod(pix, g.fd_W, ih, iw);
        xs[e] = x_qb * QX + int(cs) * p.IS + int(ih) * p.WP + int(iw);
        fdivmod(uint32_t(d_f0 + e), g.fd_P, oc, pos);
        ds[e] = xsz + d_qb * QD + int(pos) * p.OCP + int(oc);
    }
    // byte offsets: image stride, and this unit's offset in image 0 of the split
    const uint32_t x_img = uint32_t(g.IC) * g.HW * 4, d_img = uint32_t(dlen) * 4;
    const uint32_t x_vo = uint32_t(4 * x_qb) * x_img + (uint32_t(c_lo) * g.HW + x_f0) * 4;
    const uint32_t d_vo = uint32_t(4 * d_qb) * d_img + uint32_t(d_f0) * 4;
    const __amdgpu_buffer_rsrc_t xrs = tensor_rsrc(a.x, g.B * x_img);
    const __amdgpu_buffer_rsrc_t dyrs = tensor_rsrc(a.dy, g.B * d_img);
    const __amdgpu_buffer_rsrc_t ymrs = tensor_rsrc(RELU ? a.ym : a.dy, g.B * d_img);
    // raw loads of the next phase, issued by fetch() and consumed by stash()
    float4 xr[4], dr[4], mr[4];
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);

    auto fetch = [&](int ph) {
        const uint32_t b0 = uint32_t(4 * (qs + ph * p.QB));   // first image of the phase
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xr[j] = bload16(xrs, x_act ? x_vo + (b0 + j) * x_img : kOffNone);
            const uint32_t doff = d_act ? d_vo + (b0 + j) * d_img : kOffNone;
            dr[j] = bload16(dyrs, doff);
            if (RELU) mr[j] = bload16(ymrs, doff);
        }
    };
    auto stash = [&](int buf) {
        float4 *base = lds4w + buf * p.bufsz;
        if (x_act) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                base[xs[e]] = make_float4(comp(xr[0], e), comp(xr[1], e), comp(xr[2], e), comp(xr[3], e));
        }
        if (d_act) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float de[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    de[j] = comp(dr[j], e);
                    if (RELU && !(comp(mr[j], e) > 0.f)) de[j] = 0.f;
                }
                base[ds[e]] = make_float4(de[0], de[1], de[2], de[3]);
            }
        }
    };

    // this wave's 16-row oc block and column blocks
    const bool wave_on = !loader && wave < p.MBLK * p.WN;
    const int mblk = wave % p.MBLK, nsub = wave / p.MBLK;
    const int oc_a = mblk * 16 + (lane & 15);            // A row of this lane
    int coloff[NBWV];
    bool ones[NBWV];      // the bias column: B is 1 for every image
#pragma unroll
    for (int nb = 0; nb < NBWV; ++nb) {
        const int col = col0 + (nsub * NBWV + nb) * 16 + (lane & 15);
        ones[nb] = BIAS && col == g.K;
        coloff[nb] = 0;
        if (col < g.K) {
            uint32_t ic, t, kh, kw;
            fdivmod(uint32_t(col), g.fd_KK, ic, t);
            fdivmod(t, g.fd_KW, kh, kw);
            coloff[nb] = (int(ic) - c_lo) * p.IS + int(kh) * p.WP + int(kw);
        }
    }
    // per 4-step block: LDS slots of this lane's x pixel and dz element
    int xrow[kSppMax], drow[kSppMax];
#pragma unroll
    for (int s = 0; s < kSppMax; ++s) {
        const int t = 4 * s + (lane >> 4);
        xrow[s] = 0;
        drow[s] = zslot;
        if (s < p.SPP && t < p.QB * g.P) {
            uint32_t qb, pos, oh, ow;
            fdivmod(uint32_t(t), g.fd_P, qb, pos);
            fdivmod(pos, g.fd_OW, oh, ow);
            xrow[s] = int(qb) * QX + int(oh) * g.S * p.WP + int(ow) * g.S;
            if (oc_a < g.OC) drow[s] = xsz + int(qb) * QD + int(pos) * p.OCP + oc_a;
        }
    }

    f32x4 acc[NBWV];
#pragma unroll
    for (int nb = 0; nb < NBWV; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One barrier per phase: before it the loader waves have filled the
    // other buffer with phase ph+1 and the MFMA waves have finished reading
    // phase ph's buffer, which the loaders refill with phase ph+2 next.  The
    // roles branch outside the phase loop (each wave passes the same number
    // of barriers), so each role's registers are live only in its own loop.
    if (loader) {
        fetch(0);
        stash(0);
        if (ltid == 0) {
            lds4w[zslot] = zero4;
            lds4w[p.bufsz + zslot] = zero4;
        }
        __syncthreads();
        for (int ph = 0; ph < nph; ++ph) {
            if (ph + 1 < nph) {
                fetch(ph + 1);
                stash((ph + 1) & 1);
            }
            __syncthreads();
        }
        return;
    }
    __syncthreads();
    for (int ph = 0; ph < nph; ++ph) {
        if (wave_on) {
            const float4 *buf = lds4w + (ph & 1) * p.bufsz;
#pragma unroll
            for (int s = 0; s < kSppMax; ++s) {
                if (s < p.SPP) {
                    const float4 av = buf[drow[s]];
                    float4 bv[NBWV];
#pragma unroll
                    for (int nb = 0; nb < NBWV; ++nb)
                        bv[nb] = BIAS && ones[nb] ? make_float4(1.f, 1.f, 1.f, 1.f)
                                                  : buf[xrow[s] + coloff[nb]];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int nb = 0; nb < NBWV; ++nb)
                            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(av, j), comp(bv[nb], j),
                                                                           acc[nb], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // partial tile: C row 4*(lane/16) + v is oc, column lane%16 is k;
    // columns K+bias .. NP-1 (row padding) are written as zeros
    if (wave_on) {
        float *out = a.part + size_t(split) * g.OC * p.NP;
#pragma unroll
        for (int nb = 0; nb < NBWV; ++nb) {
            const int col = col0 + (nsub * NBWV + nb) * 16 + (lane & 15);
            if (col >= p.NP) continue;
            const bool real = col < g.K + p.bias;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int oc = mblk * 16 + 4 * (lane >> 4) + v;
                if (oc < g.OC) out[size_t(oc) * p.NP + col] = real ? acc[nb][v] : 0.f;
            }
        }
    }
}

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
        q.bufsz = q.QB * q.CCS * q.IS + q.QB * g.P * q.OCP + 1;
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
