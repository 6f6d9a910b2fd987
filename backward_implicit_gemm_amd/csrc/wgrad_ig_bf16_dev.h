// wgrad_ig_bf16_dev.h -- device code of the bf16 wgrad kernel (see
// wgrad_ig_bf16.hip): the dz regrouping pre-pass and the partial-tile kernel
// body, each as a body taking its workgroup index plus a __global__ wrapper,
// so that the fused backward (bwd_fused_bf16.hip) can run them inside its own
// launches.
#pragma once
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {


typedef unsigned short u16;

__device__ __forceinline__ uint4 ldg16(const u16 *p)
{
    uint4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

// LDS slot of pixel p in a staged x plane: every 8-pixel block takes 9
// slots.  The loader threads that store one pixel step together hold
// consecutive 8-pixel blocks; without the skip their 16-byte slots are 128
// bytes apart and every second one falls on the same four banks.
__device__ __forceinline__ int xslot(int p) { return p + (p >> 3); }

// dzg unit ((bg*PP + p)*128 + oc) = the 8 images of group bg at (oc, p),
// masked; zero for positions >= P, channels >= OC and images >= B.  One
// workgroup per (group, slice of kDzOC output channels): a slice of one image
// is contiguous in dy and y (kDzOC*P elements), so the group's 8 slices are
// copied into LDS with 16-byte loads and transposed there.
constexpr int kDzNT = 256;
constexpr int kDzOC = 32;               // output channels per workgroup
constexpr int kDzSlices = 128 / kDzOC;  // workgroups per image group
constexpr int kDzChunks = 2;            // 16-byte loads per thread per tensor: 8*kDzOC*P/8 <= 2*256
// The body for unit = group * kDzSlices + slice; the __global__ wrapper
// below runs one per workgroup.
__device__ __forceinline__ void dz_groups_bf16_body(const u16 *__restrict__ dy,
                                                    const u16 *__restrict__ ym,
                                                    uint4 *__restrict__ dzg, const Geom &g,
                                                    int relu, int PP, int unit)
{
    extern __shared__ __attribute__((aligned(16))) uint4 dz_lds[];
    const int tid = threadIdx.x;
    const int bg = unit / kDzSlices, oc0 = (unit - bg * kDzSlices) * kDzOC;
    const int nimg = min(8, g.B - bg * 8);
    const int nloc = max(0, min(kDzOC, g.OC - oc0));   // real channels of the slice
    const int per = g.OC * g.P;                      // elements per image
    const int L = nloc * g.P;                        // contiguous elements per image slice
    const int LS = kDzOC * g.P;                      // LDS stride of an image slice
    const uint32_t base = uint32_t(bg) * 8 * per + uint32_t(oc0) * g.P;
    u16 *sdy = reinterpret_cast<u16 *>(dz_lds);      // [8][LS]
    u16 *sym = sdy + 8 * LS;
    if ((L & 7) == 0) {
        const int per8 = L >> 3, tot = nimg * per8;
        uint4 vd[kDzChunks], vm[kDzChunks];
#pragma unroll
        for (int k = 0; k < kDzChunks; ++k) {
            const int c = tid + k * kDzNT;
            vd[k] = vm[k] = make_uint4(0, 0, 0, 0);
            if (c < tot) {
                const int i = c / per8, e = 8 * (c - i * per8);
                vd[k] = ldg16(dy + base + uint32_t(i) * per + e);
                if (relu) vm[k] = ldg16(ym + base + uint32_t(i) * per + e);
            }
        }
#pragma unroll
        for (int k = 0; k < kDzChunks; ++k) {
            const int c = tid + k * kDzNT;
            if (c < tot) {
                const int i = c / per8, e = 8 * (c - i * per8);
                __builtin_memcpy(sdy + i * LS + e, &vd[k], 16);
                __builtin_memcpy(sym + i * LS + e, &vm[k], 16);
            }
        }
    } else {
        for (int c = tid; c < nimg * L; c += kDzNT) {
            const int i = c / L, e = c - i * L;
            sdy[i * LS + e] = dy[base + uint32_t(i) * per + e];
            sym[i * LS + e] = relu ? ym[base + uint32_t(i) * per + e] : u16(0);
        }
    }
    __syncthreads();
    for (int u = tid; u < PP * kDzOC; u += kDzNT) {
        const int p = u / kDzOC, ol = u - p * kDzOC;
        u16 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            u16 d = 0;
            if (i < nimg && p < g.P && ol < nloc) {
                const int e = i * LS + ol * g.P + p;
                d = sdy[e];
                if (relu && uint32_t(sym[e]) - 1u >= 0x7F80u) d = 0;   // keep where 0 < y <= +inf
            }
            v[i] = d;
        }
        uint4 o;
        o.x = v[0] | (uint32_t(v[1]) << 16);
        o.y = v[2] | (uint32_t(v[3]) << 16);
        o.z = v[4] | (uint32_t(v[5]) << 16);
        o.w = v[6] | (uint32_t(v[7]) << 16);
        dzg[(uint32_t(bg) * PP + p) * 128 + oc0 + ol] = o;
    }
}
// LDS bytes of one regrouping workgroup
inline size_t dz_groups_lds(const Geom &g) { return size_t(2) * 8 * kDzOC * g.P * sizeof(u16); }
__global__ void __launch_bounds__(kDzNT) __attribute__((unused)) dz_groups_bf16(const u16 *__restrict__ dy,
                                                        const u16 *__restrict__ ym,
                                                        uint4 *__restrict__ dzg, Geom g, int relu,
                                                        int PP)
{
    dz_groups_bf16_body(dy, ym, dzg, g, relu, PP, blockIdx.x);
}

struct WgradBfArgs {
    Geom g;
    const u16 *x;
    const uint4 *dzg;
    float *part;
    WgradBfPlan p;
};

constexpr int kWgNT = 512;     // 8 waves

// One stage of staged operands in registers: the x unit of this thread
// (4 images x 8 pixels of one channel) and its NSTEP dz units (a stage of
// dz is PP*128 = NSTEP*512 units of 16 bytes).
template <int NSTEP>
struct WgStage {
    uint4 x[4];
    uint4 d[NSTEP];
};

// The kernel body for workgroup `bid` of the grid laid out below.
template <int NSTEP>
__device__ __forceinline__ void wgrad_ig_bf16_body(const WgradBfArgs &a, int bid)
{
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    const WgradBfPlan &p = a.p;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1;          // output channels 64*wm .. +63
    const int wn = wave >> 1;         // columns 32*wn .. +31 of the tile
    const int N = g.K;                // IC*KH*KW columns
    // Workgroups are dealt to the XCDs round-robin by id; ids are laid out so
    // that all column tiles of one split (one image range) share an XCD,
    // whose L2 then serves that range's dz and x to every tile.
    const int xcd = bid % g.nxcd, slot = bid / g.nxcd;
    const int split = (slot / p.ncol) * g.nxcd + xcd;
    if (split >= p.splits) return;
    const int n0 = (slot % p.ncol) * 128;
    const int c_lo = n0 / g.KK;
    const int gb = split * p.gps;
    const int ge = min(gb + p.gps, p.ngroups);

    const int xbuf = p.CCW * p.HWP;               // 16-byte units per x stage
    const int dbuf = p.PP * 128;                  // 16-byte units per dz stage
    uint4 *xs = lds4;                             // [2][CCW][HWP]
    uint4 *ds = lds4 + 2 * xbuf;                  // [2][PP][128]

    // ---- per-lane fragment offsets (16-byte units) -------------------------
    // B (x): column n = n0 + 32*wn + 16*j + lane%16 -> (ic, kh, kw); position
    // p = 4*s + lane/16 -> pixel (oh*S, ow*S).  Padded columns and positions
    // read a valid pixel; their dz is zero or their result is not stored.
    int xcol[2], xpl[2], xrow[NSTEP], drow[NSTEP];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = min(n0 + 32 * wn + 16 * j + (lane & 15), N - 1);
        uint32_t ic, kk, kh, kw;
        fdivmod(uint32_t(n), g.fd_KK, ic, kk);
        fdivmod(kk, g.fd_KW, kh, kw);
        xpl[j] = (int(ic) - c_lo) * p.HWP;
        xcol[j] = int(kh) * g.W + int(kw);
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const int pp = 4 * s + (lane >> 4);
        const int pc = min(pp, g.P - 1);
        uint32_t oh, ow;
        fdivmod(uint32_t(pc), g.fd_OW, oh, ow);
        xrow[s] = int(oh) * g.S * g.W + int(ow) * g.S;
        drow[s] = pp * 128 + 64 * wm + (lane & 15);
    }
    int xoff[2][NSTEP];      // LDS slot of this lane's B value per column block and step
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) xoff[j][s] = xpl[j] + xslot(xcol[j] + xrow[s]);

    // ---- staging -----------------------------------------------------------
    // x unit (icl, blk, half): pixels [pix, pix+8) of channel c_lo + icl for
    // images 4*half .. 4*half+3 of the group, pix = min(8*blk, HW-8) so every
    // 16-byte load stays inside its plane (the last block overlaps its
    // neighbour and rewrites the same values).  Every thread issues the same
    // loads, from clamped valid addresses where it has no unit, so the wait
    // for a stage is an exact count of the loads issued after it.  Images
    // past the batch are zeroed (their dz is zero too; a zero x keeps
    // non-finite values out of the sums).
    const bool xon = tid < 2 * p.CCW * p.nblk;
    const int xunit = xon ? tid >> 1 : 0;
    const int xhalf = tid & 1;
    const int xicl = xunit / p.nblk;
    const int xpix = min(8 * (xunit - xicl * p.nblk), g.HW - 8);
    const int xic = min(c_lo + xicl, g.IC - 1);
    auto fetch = [&](int grp, WgStage<NSTEP> &st) {
        const int b0 = grp * 8 + 4 * xhalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = min(b0 + i, g.B - 1);
            st.x[i] = ldg16(a.x + (uint32_t(b) * g.IC + xic) * g.HW + xpix);
        }
        const uint4 *src = a.dzg + size_t(grp) * dbuf;
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) st.d[k] = src[tid + k * kWgNT];
    };
    auto stash = [&](int grp, const WgStage<NSTEP> &st, int buf) {
        if (xon) {
            const int nb = g.B - grp * 8 - 4 * xhalf;   // images of this half in the batch
            uint32_t in[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = i < nb;
                in[i][0] = ok ? st.x[i].x : 0u; in[i][1] = ok ? st.x[i].y : 0u;
                in[i][2] = ok ? st.x[i].z : 0u; in[i][3] = ok ? st.x[i].w : 0u;
            }
            // pixel pp's 16-byte slot holds images 0..7; this thread writes
            // the 8 bytes of its four: word j = images (2j, 2j+1)
            uint4 *plane = xs + buf * xbuf + xicl * p.HWP;
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) {
                const int wi = pp >> 1;
                uint32_t o[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t lo = in[2 * j][wi], hi = in[2 * j + 1][wi];
                    o[j] = (pp & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
                }
                reinterpret_cast<uint2 *>(plane + xslot(xpix + pp))[xhalf] = make_uint2(o[0], o[1]);
            }
        }
        uint4 *dd = ds + buf * dbuf;
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) dd[tid + k * kWgNT] = st.d[k];
    };

    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mfma_stage = [&](int buf) {
        const uint4 *xb = xs + buf * xbuf;
        const uint4 *db = ds + buf * dbuf;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = __builtin_bit_cast(bf16x8, db[drow[s] + 16 * i]);
#pragma unroll
            for (int j = 0; j < 2; ++j) bfr[j] = __builtin_bit_cast(bf16x8, xb[xoff[j][s]]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    // Pipeline: stage i's operands sit in LDS buffer i&1 while stage i+1's
    // are in registers and stage i+2's loads are in flight.  The register
    // slots alternate, so the loop body is written out twice.
    WgStage<NSTEP> r0, r1;
    const int ng = ge - gb;
    if (ng > 0) fetch(gb, r0);
    if (ng > 1) fetch(gb + 1, r1);
    if (ng > 0) stash(gb, r0, 0);
    __syncthreads();
    for (int i = 0; i < ng; i += 2) {
        // stage i (LDS 0); r1 holds stage i+1; r0 is free
        if (i + 2 < ng) fetch(gb + i + 2, r0);
        mfma_stage(0);
        if (i + 1 >= ng) break;
        stash(gb + i + 1, r1, 1);
        __syncthreads();
        // stage i+1 (LDS 1); r0 holds stage i+2; r1 is free
        if (i + 3 < ng) fetch(gb + i + 3, r1);
        mfma_stage(1);
        if (i + 2 >= ng) break;
        stash(gb + i + 2, r0, 0);
        __syncthreads();
    }

    // ---- partial tile: lane holds rows 4*(lane/16) + v of column lane%16 ----
    float *part = a.part + size_t(split) * g.OC * N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + 32 * wn + 16 * j + (lane & 15);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int oc = 64 * wm + 16 * i + 4 * (lane >> 4) + v;
                if (oc < g.OC) part[uint32_t(oc) * N + n] = acc[i][j][v];
            }
    }
}

// The same computation with the roles split over 16 waves: waves 0..7 run
// the MFMAs exactly as above, waves 8..15 run the staging (the same units,
// indexed by their own thread number).  A wave's vector-memory counter is in
// order, so in the 8-wave body every wait for a stage also waited for the
// loads of the stage after it; here the MFMA waves issue no global loads.
// The loaders store stage i+1 (loaded during stage i-1) into the other LDS
// buffer and issue the loads of stage i+2 while the MFMAs run stage i; one
// barrier per stage hands the buffers over.
// BIAS: the plan's bias column is computed: its lanes read their B operand
// from a unit of bf16 ones kept after each x buffer, so the MFMA loop is the
// plain one (a per-lane select there cost the plain wgrad a third of its time
// at JW = 4, and the bias variant spilled)
template <int NSTEP, int JW, bool BIAS>
__device__ __forceinline__ void wgrad_ws_bf16_body(const WgradBfArgs &a, int bid)
{
    constexpr int TW = 64 * JW;       // columns per workgroup tile
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    const WgradBfPlan &p = a.p;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool loader = wave >= 8;
    const int tid = loader ? int(threadIdx.x) - kWgNT : int(threadIdx.x);   // index within the role
    const int wm = wave & 1;          // output channels 64*wm .. +63
    const int wn = wave >> 1;         // columns 16*JW*wn .. 16*JW*wn + 16*JW-1 of the tile
    const int N = g.K;                // IC*KH*KW columns
    // Workgroups are dealt to the XCDs round-robin by id; ids are laid out so
    // that all column tiles of one split (one image range) share an XCD,
    // whose L2 then serves that range's dz and x to every tile.
    const int xcd = bid % g.nxcd, slot = bid / g.nxcd;
    const int split = (slot / p.ncol) * g.nxcd + xcd;
    if (split >= p.splits) return;
    const int n0 = (slot % p.ncol) * TW;
    // (a tile holding only the bias column stages channel IC-1, unused)
    const int c_lo = min(n0, N - 1) / g.KK;
    const int gb = split * p.gps;
    const int ge = min(gb + p.gps, p.ngroups);

    // 16-byte units per x stage; with the bias column, one more unit holding
    // bf16 ones, which the bias lanes read as their B operand
    const int xones = p.CCW * p.HWP;
    const int xbuf = xones + (BIAS ? 1 : 0);
    const int dbuf = p.PP * 128;                  // 16-byte units per dz stage
    uint4 *xs = lds4;                             // [2][CCW][HWP]
    uint4 *ds = lds4 + 2 * xbuf;                  // [2][PP][128]

    // ---- per-lane fragment offsets (16-byte units) -------------------------
    // B (x): column n = n0 + 16*JW*wn + 16*j + lane%16 -> (ic, kh, kw); position
    // p = 4*s + lane/16 -> pixel (oh*S, ow*S).  Padded columns and positions
    // read a valid pixel; their dz is zero or their result is not stored.
    int xcol[JW], xpl[JW], xrow[NSTEP], drow[NSTEP];
    bool ones[JW];        // the bias column: B is 1 for every image
#pragma unroll
    for (int j = 0; j < JW; ++j) {
        ones[j] = BIAS && n0 + 16 * JW * wn + 16 * j + (lane & 15) == N;
        const int n = min(n0 + 16 * JW * wn + 16 * j + (lane & 15), N - 1);
        uint32_t ic, kk, kh, kw;
        fdivmod(uint32_t(n), g.fd_KK, ic, kk);
        fdivmod(kk, g.fd_KW, kh, kw);
        xpl[j] = (int(ic) - c_lo) * p.HWP;
        xcol[j] = int(kh) * g.W + int(kw);
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const int pp = 4 * s + (lane >> 4);
        const int pc = min(pp, g.P - 1);
        uint32_t oh, ow;
        fdivmod(uint32_t(pc), g.fd_OW, oh, ow);
        xrow[s] = int(oh) * g.S * g.W + int(ow) * g.S;
        drow[s] = pp * 128 + 64 * wm + (lane & 15);
    }
    int xoff[JW][NSTEP];     // LDS slot of this lane's B value per column block and step
#pragma unroll
    for (int j = 0; j < JW; ++j)
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) xoff[j][s] = ones[j] ? xones : xpl[j] + xslot(xcol[j] + xrow[s]);
    if (BIAS && threadIdx.x == 0) {
        // the ones unit of both x buffers, before the first barrier
        xs[xones] = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        xs[xbuf + xones] = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    }

    // ---- staging -----------------------------------------------------------
    // x unit (icl, blk, half): pixels [pix, pix+8) of channel c_lo + icl for
    // images 4*half .. 4*half+3 of the group, pix = min(8*blk, HW-8) so every
    // 16-byte load stays inside its plane (the last block overlaps its
    // neighbour and rewrites the same values).  Every thread issues the same
    // loads, from clamped valid addresses where it has no unit, so the wait
    // for a stage is an exact count of the loads issued after it.  Images
    // past the batch are zeroed (their dz is zero too; a zero x keeps
    // non-finite values out of the sums).
    const bool xon = tid < 2 * p.CCW * p.nblk;
    const int xunit = xon ? tid >> 1 : 0;
    const int xhalf = tid & 1;
    const int xicl = xunit / p.nblk;
    const int xpix = min(8 * (xunit - xicl * p.nblk), g.HW - 8);
    const int xic = min(c_lo + xicl, g.IC - 1);
    auto fetch = [&](int grp, WgStage<NSTEP> &st) {
        const int b0 = grp * 8 + 4 * xhalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = min(b0 + i, g.B - 1);
            st.x[i] = ldg16(a.x + (uint32_t(b) * g.IC + xic) * g.HW + xpix);
        }
        const uint4 *src = a.dzg + size_t(grp) * dbuf;
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) st.d[k] = src[tid + k * kWgNT];
    };
    auto stash = [&](int grp, const WgStage<NSTEP> &st, int buf) {
        if (xon) {
            const int nb = g.B - grp * 8 - 4 * xhalf;   // images of this half in the batch
            uint32_t in[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = i < nb;
                in[i][0] = ok ? st.x[i].x : 0u; in[i][1] = ok ? st.x[i].y : 0u;
                in[i][2] = ok ? st.x[i].z : 0u; in[i][3] = ok ? st.x[i].w : 0u;
            }
            // pixel pp's 16-byte slot holds images 0..7; this thread writes
            // the 8 bytes of its four: word j = images (2j, 2j+1)
            uint4 *plane = xs + buf * xbuf + xicl * p.HWP;
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) {
                const int wi = pp >> 1;
                uint32_t o[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t lo = in[2 * j][wi], hi = in[2 * j + 1][wi];
                    o[j] = (pp & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
                }
                reinterpret_cast<uint2 *>(plane + xslot(xpix + pp))[xhalf] = make_uint2(o[0], o[1]);
            }
        }
        uint4 *dd = ds + buf * dbuf;
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) dd[tid + k * kWgNT] = st.d[k];
    };

    f32x4 acc[4][JW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mfma_stage = [&](int buf) {
        const uint4 *xb = xs + buf * xbuf;
        const uint4 *db = ds + buf * dbuf;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            bf16x8 af[4], bfr[JW];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = __builtin_bit_cast(bf16x8, db[drow[s] + 16 * i]);
#pragma unroll
            for (int j = 0; j < JW; ++j) bfr[j] = __builtin_bit_cast(bf16x8, xb[xoff[j][s]]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < JW; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    const int ng = ge - gb;
    if (loader) {
        WgStage<NSTEP> r;
        if (ng > 0) {
            fetch(gb, r);
            stash(gb, r, 0);
        }
        if (ng > 1) fetch(gb + 1, r);
        __syncthreads();
        for (int i = 0; i < ng; ++i) {
            if (i + 1 < ng) {
                stash(gb + i + 1, r, (i + 1) & 1);
                if (i + 2 < ng) fetch(gb + i + 2, r);
            }
            __syncthreads();
        }
        return;
    }
    __syncthreads();
    for (int i = 0; i < ng; ++i) {
        mfma_stage(i & 1);
        __syncthreads();
    }

    // ---- partial tile: lane holds rows 4*(lane/16) + v of column lane%16 ----
    // columns K+bias .. NP-1 (row padding) are written as zeros
    float *part = a.part + size_t(split) * g.OC * p.NP;
#pragma unroll
    for (int j = 0; j < JW; ++j) {
        const int n = n0 + 16 * JW * wn + 16 * j + (lane & 15);
        if (n >= p.NP) continue;
        const bool real = n < N + p.bias;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int oc = 64 * wm + 16 * i + 4 * (lane >> 4) + v;
                if (oc < g.OC) part[uint32_t(oc) * p.NP + n] = real ? acc[i][j][v] : 0.f;
            }
    }
}

template <int NSTEP>
__global__ void __launch_bounds__(kWgNT) wgrad_ig_bf16(WgradBfArgs a)
{
    wgrad_ig_bf16_body<NSTEP>(a, blockIdx.x);
}

template <int NSTEP, int JW, bool BIAS>
__global__ void __launch_bounds__(2 * kWgNT) wgrad_ws_bf16(WgradBfArgs a)
{
    wgrad_ws_bf16_body<NSTEP, JW, BIAS>(a, blockIdx.x);
}

}  // namespace
}  // namespace gc
