// fwd_pack.hip -- pieces shared by the two forward kernels (fwd_ws_bf16.hip,
// fwd_ws_f32.hip): the per-call weight packing into MFMA B-fragment order and
// the LDS pitch choice of the channels-innermost x tile.
//
// Both forwards order the reduction index (channel group, tap, channel in the
// group), so that a lane's MFMA operand is a run of consecutive channels at one
// tap: 8 channels (16 bytes) for v_mfma_f32_16x16x32_bf16, 4 channels (16
// bytes) for v_mfma_f32_16x16x4_f32 (whose steps may also share one tap
// among four channel groups, see FwdF32Steps).  OIHW weights hold a tap's
// channels KH*KW elements apart, so a small pass per call gathers them into
// fragment order, padding channels and taps with zeros; each wave then
// streams its fragments as contiguous 1 KB reads.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

typedef unsigned short u16;

// Packed weight layout, 16-byte units: ((nb*NCG + cg)*TS + s)*64 + lane,
// lane = (n%16) + 16*q, holding w[n][8*cg + i][4*s + q] for i = 0..7 (zero
// past OC, IC or KH*KW).  Block nb is blockIdx.y; fd_ts divides by TS.
__global__ void __launch_bounds__(256) pack_w_fwd_bf16(const u16 *__restrict__ w,
                                                       uint4 *__restrict__ wf, Geom g, int NCG,
                                                       FastDiv fd_ts)
{
    const int nb = blockIdx.y;
    const int per_block = NCG * int(fd_ts.d) * 64;
    const int u = blockIdx.x * 256 + threadIdx.x;      // unit within the block
    if (u >= per_block) return;
    const int lane = u & 63;
    uint32_t cg, s;
    fdivmod(uint32_t(u >> 6), fd_ts, cg, s);
    const int n = nb * 16 + (lane & 15);
    const int t = 4 * int(s) + (lane >> 4);
    u16 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ic = 8 * int(cg) + i;
        v[i] = (n < g.OC && ic < g.IC && t < g.KK) ? w[(size_t(n) * g.IC + ic) * g.KK + t] : u16(0);
    }
    uint4 o;
    o.x = v[0] | (uint32_t(v[1]) << 16);
    o.y = v[2] | (uint32_t(v[3]) << 16);
    o.z = v[4] | (uint32_t(v[5]) << 16);
    o.w = v[6] | (uint32_t(v[7]) << 16);
    wf[size_t(nb) * per_block + u] = o;
}

// Packed fp32 weights, 16-byte units (nb*NFRAG + f)*64 + lane: step f of
// block nb (FwdF32Steps order), lane = n%16 + 16*q, holding four consecutive
// channels of column n = 16*nb + lane%16 at one tap: for a full step (group
// cg, tap step s) channels 4*cg .. 4*cg+3 at tap 4*s + q; for a shared step l
// of a phase, channels of group 4*l + q of the phase at the last tap.  Zero
// past OC, IC or KH*KW, and for lane groups past the phase's groups.
// Block nb is blockIdx.y.  Every phase but the last has nsteps(0) steps, so
// the phase of step f is min(f / nsteps(0), nph - 1); the two divisions use
// divisors prepared on the host.
__global__ void __launch_bounds__(256) pack_w_fwd_f32(const float *__restrict__ w,
                                                      float4 *__restrict__ wf, Geom g,
                                                      FwdF32Steps st, FastDiv fd_ns0,
                                                      FastDiv fd_tsf)
{
    const int nfrag = st.nfrag();
    const int nb = blockIdx.y;
    const int u = blockIdx.x * 256 + threadIdx.x;      // unit within the block
    if (u >= nfrag * 64) return;
    const int lane = u & 63, q = lane >> 4;
    int f = u >> 6;
    const int ph = min(int(fdiv(uint32_t(f), fd_ns0)), st.nph() - 1);
    f -= ph * st.nsteps(0);
    int cg, t;
    bool ok;
    if (f < st.nfull(ph)) {
        uint32_t s, tq;
        fdivmod(uint32_t(f), fd_tsf, s, tq);
        cg = ph * st.CPP + int(s);
        t = 4 * int(tq) + q;
        ok = true;
    } else {
        const int l = f - st.nfull(ph);
        cg = ph * st.CPP + 4 * l + q;
        t = g.KK - 1;
        ok = 4 * l + q < st.ncg(ph);
    }
    const int n = nb * 16 + (lane & 15);
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ic = 4 * cg + j;
        v[j] = (ok && n < g.OC && ic < g.IC && t < g.KK) ? w[(size_t(n) * g.IC + ic) * g.KK + t] : 0.f;
    }
    wf[size_t(nb) * nfrag * 64 + u] = make_float4(v[0], v[1], v[2], v[3]);
}

}  // namespace

// LDS pitch of the channels-innermost x tile.  A 16-lane group of an A
// fragment read fetches the 16-byte pixel slots of 16 output rows at one
// tap; the LDS serves it in one pass only if the 16 slots fall in distinct
// 16-byte bank groups (slot mod 16).  Pad the row pitch WP and the image
// stride IS (each by less than 16 slots) to minimise the worst-case
// multiplicity summed over every row block and tap.
static void search_lds_pitch(const Geom &g, int G, int MB, int TS, int &WP_out, int &IS_out)
{
    int best = 1 << 30;
    WP_out = g.W;
    IS_out = g.H * g.W;
    const int rows = G * g.P;
    for (int WP = g.W; WP < g.W + 16; ++WP)
        for (int IS = g.H * WP; IS < g.H * WP + 16; ++IS) {
            int cost = 0;
            for (int mb = 0; mb < MB; ++mb)
                for (int t = 0; t < std::min(4 * TS, g.KK); ++t) {
                    int cnt[16] = {0}, worst = 0;
                    for (int l = 0; l < 16; ++l) {
                        const int r = mb * 16 + l;
                        int slot = 0;
                        if (r < rows) {
                            const int img = r / g.P, pp = r % g.P;
                            slot = img * IS + (pp / g.OW) * g.S * WP + (pp % g.OW) * g.S;
                        }
                        slot += (t / g.KW) * WP + t % g.KW;
                        worst = std::max(worst, ++cnt[slot & 15]);
                    }
                    cost += worst;
                }
            // fewer conflicts first, then the smaller tile
            if (cost < best) {
                best = cost;
                WP_out = WP;
                IS_out = IS;
            }
        }
}

// The search does not depend on the batch size beyond the rows G*P the
// images fill, so it runs once per layer shape and G.
void pick_lds_pitch(const Geom &g, int G, int MB, int TS, int &WP_out, int &IS_out)
{
    static SearchMemo<std::pair<int, int>> memo;
    const int key[12] = {g.IC, g.H, g.W, g.OC, g.KH, g.KW, g.S, G, MB, TS, 0, 0};
    const std::pair<int, int> r = memo.get(key, [&] {
        int wp = 0, is = 0;
        search_lds_pitch(g, G, MB, TS, wp, is);
        return std::make_pair(wp, is);
    });
    WP_out = r.first;
    IS_out = r.second;
}

hipError_t launch_pack_w_fwd_bf16(const Geom &g, int NCG, int TS, int nblocks, const void *w,
                                  void *wf, size_t ws_bytes, hipStream_t s)
{
    const int per_block = NCG * TS * 64;
    if (TS < 1 || size_t(nblocks) * per_block * 16 > ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_fwd_bf16, dim3((per_block + 255) / 256, nblocks), dim3(256), 0, s,
                       (const u16 *)w, (uint4 *)wf, g, NCG, make_fastdiv(TS));
    return hipGetLastError();
}

hipError_t launch_pack_w_fwd_f32(const Geom &g, int NCG, int CPP, int TS, int lo, int nblocks,
                                 const void *w, void *wf, size_t ws_bytes, hipStream_t s)
{
    const FwdF32Steps st{NCG, CPP, TS, lo};
    if (CPP < 1 || TS < 1 || (lo && (TS < 2 || g.KK != 4 * (TS - 1) + 1))) return hipErrorInvalidValue;
    const int per_block = st.nfrag() * 64;
    if (size_t(nblocks) * per_block * 16 > ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_fwd_f32, dim3((per_block + 255) / 256, nblocks), dim3(256), 0, s,
                       (const float *)w, (float4 *)wf, g, st, make_fastdiv(st.nsteps(0)),
                       make_fastdiv(st.tsf()));
    return hipGetLastError();
}

}  // namespace gc
