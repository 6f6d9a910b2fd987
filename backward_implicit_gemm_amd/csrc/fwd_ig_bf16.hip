// fwd_ig_bf16.hip -- forward convolution, bf16 storage, fp32 accumulation.
//
// Implicit GEMM y[m][n] = sum_k A[m][k] * w[n][k], m = (b,oh,ow), n = oc,
// on v_mfma_f32_16x16x32_bf16, whose operands carry 8 consecutive reduction
// elements per lane.  The reduction index is ordered (channel group of 8,
// tap, channel within the group) so that both operands are single 16-byte
// reads:
//   * x: a workgroup owns G whole images; each channel group of the images is
//     staged in LDS channels-innermost, [image][pixel][8 channels], so the A
//     fragment of output row (b,oh,ow) and tap (kh,kw) is the 16 bytes at
//     pixel (oh*S+kh, ow*S+kw).  The transposition from NCHW happens in
//     registers (8 pixels x 8 channels per thread) before ds_write_b128.
//   * w: a small pre-pass packs the weights into the exact fragment order the
//     MFMAs consume -- [16-channel block][channel group][tap step][lane][8] --
//     so each wave's B fragment for one step is one contiguous 1 KB read,
//     streamed from L2 straight into a ring of registers 16 fragments ahead
//     (the MFMA work per fragment is far shorter than an L2 round trip).  The
//     fragment sequence is unrolled at compile time (one instantiation per
//     channel-group count), which keeps the ring in fixed registers; shapes
//     without an instantiation use the shape-generic kernel.
// Channels are padded to a multiple of 8 and taps to a multiple of 4 with
// zero weights.  The whole x tile of the workgroup (all channel groups) is
// staged into LDS in NPH phases, each phase's global loads in flight while
// the previous phase's MFMAs run.  Epilogue: optional ReLU, round-to-nearest-even to
// bf16, NCHW store.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

typedef unsigned short u16;

// Packed weight layout, 16-byte units: ((nb*NCG + cg)*TS + s)*64 + lane,
// lane = (n%16) + 16*q, holding w[n][8*cg + i][4*s + q] for i = 0..7 (zero
// past OC, IC or KH*KW).
__global__ void __launch_bounds__(256) pack_w_fwd_bf16(const u16 *__restrict__ w,
                                                       uint4 *__restrict__ wf, Geom g, int NCG,
                                                       int TS, int total)
{
    for (int u = blockIdx.x * 256 + threadIdx.x; u < total; u += gridDim.x * 256) {
        const int lane = u & 63;
        int rest = u >> 6;
        const int s = rest % TS;
        rest /= TS;
        const int cg = rest % NCG;
        const int nb = rest / NCG;
        const int n = nb * 16 + (lane & 15);
        const int t = 4 * s + (lane >> 4);
        u16 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ic = 8 * cg + i;
            v[i] = (n < g.OC && ic < g.IC && t < g.KK) ? w[(size_t(n) * g.IC + ic) * g.KK + t] : u16(0);
        }
        uint4 o;
        o.x = v[0] | (uint32_t(v[1]) << 16);
        o.y = v[2] | (uint32_t(v[3]) << 16);
        o.z = v[4] | (uint32_t(v[5]) << 16);
        o.w = v[6] | (uint32_t(v[7]) << 16);
        wf[u] = o;
    }
}

struct FwdBfArgs {
    Geom g;
    const u16 *x;
    const uint4 *wf;
    const u16 *bias;
    u16 *y;
    int relu;
    int G;        // images per workgroup
    int WP;       // LDS pixel slots per image row (>= W)
    int IS;       // LDS pixel slots per image (>= H*WP)
    int NCG;      // channel groups of 8
    int nblk;     // 8-pixel blocks per image plane
};

// 16 bytes from a 2-byte-aligned global address (one global_load_dwordx4).
__device__ __forceinline__ uint4 ldg16_any(const u16 *p)
{
    uint4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

template <int NW, int MB, int TS, int NCG, int NPH, int D>
__global__ void __launch_bounds__(64 * NW) fwd_ig_bf16(FwdBfArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    constexpr int NT = 64 * NW;
    constexpr int BN = 16 * NW;
    constexpr int NFRAG = NCG * TS;
    constexpr int CPP = (NCG + NPH - 1) / NPH;       // channel groups per staging phase
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b0 = blockIdx.x * a.G;
    const int gimg = min(a.G, g.B - b0);
    const int rows = gimg * g.P;
    const int n0 = blockIdx.y * BN;
    const int nb = blockIdx.y * NW + wave;           // 16-channel block of this wave
    const int gstride = a.G * a.IS;                  // uint4 per channel group in LDS

    uint4 *xs = lds4;                                // [NCG][G][IS] x 8 channels

    // Weight fragments stream from L2 through a ring of D registers per lane:
    // fragment f = cg*TS + s is consumed at step f and its slot refilled with
    // fragment f + D.  Everything below is unrolled at compile time, so the
    // ring stays in fixed registers and each use waits only for its own load.
    const uint4 *wf_wave = a.wf + size_t(nb) * NFRAG * 64 + lane;
    uint4 ring[D];
#pragma unroll
    for (int j = 0; j < D; ++j)
        ring[j] = j < NFRAG ? wf_wave[size_t(j) * 64] : make_uint4(0, 0, 0, 0);

    // x staging, one unit per thread per phase: unit u = (cg, img, 8-pixel
    // block) of the phase's channel groups; 8 loads of 8 pixels (one per
    // channel), an 8x8 register transpose, 8 stores of 8 channels (channels
    // innermost).  The loads are buffer loads without branches, so they stay
    // in flight through the phase's MFMAs: channels past IC and images past
    // the batch use an offset past the end of x and read zeros, and the last
    // block of a plane is moved back to end with it (HW >= 8), rewriting some
    // of its neighbour's slots with the same values.  Every LDS slot an MFMA
    // reads is written (row and image padding slots are never read).
    const int units_per_cg = a.G * a.nblk;
    const int u_blk = tid % a.nblk, u_img = (tid / a.nblk) % a.G, u_cgl = tid / units_per_cg;
    const int u_w0 = min(8 * u_blk, g.HW - 8);
    const bool u_img_ok = u_img < gimg;
    const uint32_t plane_bytes = uint32_t(g.HW) * 2;
    const uint32_t u_off = (uint32_t(b0 + u_img) * g.IC * g.HW + u_w0) * 2;
    const __amdgpu_buffer_rsrc_t xrs = tensor_rsrc(a.x, uint32_t(g.B) * g.IC * plane_bytes);
    uint32_t in[8][4];
    int u_cg = 0;
    bool u_on = false;
    auto fetch_x = [&](int ph) {
        const int cg0 = ph * CPP;
        const int ncg = min(CPP, NCG - cg0);
        u_on = u_cgl < ncg;
        u_cg = cg0 + u_cgl;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ic = u_cg * 8 + c;
            const uint4 v = bload16u(xrs, u_on && u_img_ok && ic < g.IC ? u_off + uint32_t(ic) * plane_bytes
                                                                       : kOffNone);
            in[c][0] = v.x; in[c][1] = v.y; in[c][2] = v.z; in[c][3] = v.w;
        }
    };
    auto stash_x = [&]() {
        if (!u_on) return;
        // word j of pixel p = channels (2j, 2j+1) at pixel p; pixel (ih, iw)
        // lives in slot ih*WP + iw of its image
        uint4 *dst = xs + u_cg * gstride + u_img * a.IS;
        int ih = u_w0 / g.W, iw = u_w0 - ih * g.W;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int wi = pp >> 1;
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo_src = in[2 * j][wi], hi_src = in[2 * j + 1][wi];
                o[j] = (pp & 1) ? ((lo_src >> 16) | (hi_src & 0xFFFF0000u))
                                : ((lo_src & 0xFFFFu) | (hi_src << 16));
            }
            dst[ih * a.WP + iw] = make_uint4(o[0], o[1], o[2], o[3]);
            if (++iw == g.W) { iw = 0; ++ih; }
        }
    };

    // LDS pixel offsets (16-byte units) of this lane's A rows and taps.
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
    int toff[TS];
#pragma unroll
    for (int s = 0; s < TS; ++s) {
        const int t = 4 * s + (lane >> 4);
        toff[s] = 0;
        if (t < g.KK) {
            uint32_t kh, kw;
            fdivmod(t, g.fd_KW, kh, kw);
            toff[s] = int(kh) * a.WP + int(kw);
        }
    }

    f32x4 acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    fetch_x(0);
    stash_x();
    __syncthreads();
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        if (ph + 1 < NPH) fetch_x(ph + 1);       // next phase's loads fly during this one
#pragma unroll
        for (int cg = ph * CPP; cg < (ph + 1) * CPP && cg < NCG; ++cg) {
            // all A fragments of the channel group first, so the LDS latency
            // overlaps; then the group's MFMAs
            const uint4 *xb = xs + cg * gstride;
            uint4 af[TS][MB];
#pragma unroll
            for (int st = 0; st < TS; ++st)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) af[st][mb] = xb[rowoff[mb] + toff[st]];
#pragma unroll
            for (int st = 0; st < TS; ++st) {
                const int f = cg * TS + st;
                const bf16x8 bv = __builtin_bit_cast(bf16x8, ring[f % D]);
                if (f + D < NFRAG) ring[f % D] = wf_wave[size_t(f + D) * 64];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[st][mb]), bv, acc[mb], 0, 0, 0);
            }
        }
        if (ph + 1 < NPH) {
            stash_x();
            __syncthreads();
        }
    }

    // epilogue: row r = mb*16 + 4*(lane/16) + v, column n0 + wave*16 + lane%16
    const int n = n0 + wave * 16 + (lane & 15);
    if (n < g.OC) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = mb * 16 + (lane >> 4) * 4 + v;
                if (r >= rows) continue;
                uint32_t img, pp;
                fdivmod(r, g.fd_P, img, pp);
                float val = acc[mb][v];
                if (a.bias) val += __uint_as_float(uint32_t(a.bias[n]) << 16);
                if (a.relu && !(val > 0.f)) val = 0.f;
                a.y[(size_t(b0 + int(img)) * g.OC + n) * g.P + int(pp)] = from_f32<bf16_t>(val);
            }
    }
}

struct FwdBfVariant {
    int NW, MB, TS, NCG, NPH;
    void (*fn)(FwdBfArgs);
};

constexpr int kRing = 16;   // weight fragments in flight per lane
#define FB_V(NW, MB, TS, NCG, NPH) {NW, MB, TS, NCG, NPH, fwd_ig_bf16<NW, MB, TS, NCG, NPH, kRing>}
const FwdBfVariant kFwdBfVariants[] = {
    FB_V(8, 3, 7, 8, 2),    // layer 1: 4 images x 12 rows, 25 taps (7 steps), 59 -> 64 channels
    FB_V(8, 1, 7, 8, 1),    // layer 1, fewer than 4 images per workgroup
    FB_V(4, 1, 3, 16, 1),   // layer 2: 8 images x 2 rows, 9 taps (3 steps), 128 channels
    FB_V(4, 4, 3, 16, 4),   // layer 2 at large batch: 32 images
    FB_V(4, 2, 3, 16, 2), FB_V(4, 3, 3, 16, 4),
    FB_V(8, 1, 2, 2, 1),    // 13 channels, 3x2 kernel (odd-shape test)
};
#undef FB_V

// A variant whose staging phases give every unit a thread: NPH phases of
// ceil(NCG/NPH) channel groups x G images x nblk pixel blocks each.
const FwdBfVariant *pick_fwd_bf(int NW, int MB, int TS, int NCG, int units_per_cg)
{
    for (const auto &v : kFwdBfVariants)
        if (v.NW == NW && v.MB == MB && v.TS == TS && v.NCG == NCG &&
            (NCG + v.NPH - 1) / v.NPH * units_per_cg <= 64 * NW)
            return &v;
    return nullptr;
}

}  // namespace

// LDS pitch of the channels-innermost x tile.  A 16-lane group of an A
// fragment read fetches the 16-byte pixel slots of 16 output rows at one
// tap; the LDS serves it in one pass only if the 16 slots fall in distinct
// 16-byte bank groups (slot mod 16).  Pad the row pitch WP and the image
// stride IS (each by less than 16 slots) to minimise the worst-case
// multiplicity summed over every row block and tap.
void pick_lds_pitch(const Geom &g, int G, int MB, int TS, int &WP_out, int &IS_out)
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

bool plan_fwd_ig_bf16(const Geom &g, FwdBfPlan &p)
{
    if (g.P > 64 || g.KK > 36) return false;
    // staging windows of 8 pixels inside a plane; x addressed by 32-bit
    // buffer offsets
    if (g.HW < 8 || size_t(g.B) * g.IC * g.HW * 2 >= (size_t(1) << 31)) return false;
    const int TS = (g.KK + 3) / 4;
    // Few rows per image (layer-2-like): 4 waves and twice the images, so each
    // workgroup streams half the weights for twice the rows.
    const int order[2] = {g.P <= 4 ? 4 : 8, g.P <= 4 ? 8 : 4};
    for (int NW : order) {
        const int BN = 16 * NW;
        const int ntile_n = (g.OC + BN - 1) / BN;
        int G = std::max(1, 64 / g.P);
        while (G > 1 && ((g.B + G - 1) / G) * ntile_n < 256) --G;
        if (g.P == 12 && G > 4) G = 4;
        if (G > g.B) G = g.B;
        const int MB = (G * g.P + 15) / 16;
        FwdBfPlan q;
        q.NW = NW; q.G = G; q.MB = MB; q.TS = TS;
        q.nblk = (g.HW + 7) / 8;
        q.NCG = (g.IC + 7) / 8;
        pick_lds_pitch(g, G, MB, TS, q.WP, q.IS);
        q.lds = sizeof(uint4) * size_t(q.NCG) * G * q.IS;   // the whole x tile
        if (q.lds > 150 * 1024) continue;
        if (!pick_fwd_bf(NW, MB, TS, q.NCG, G * q.nblk)) continue;
        // packed weights for every 16-channel block a wave of the grid reads
        const int nbt_grid = ntile_n * NW;
        q.ws_bytes = size_t(nbt_grid) * q.NCG * TS * 64 * 16;
        p = q;
        return true;
    }
    return false;
}

hipError_t launch_pack_w_fwd_bf16(const Geom &g, int NCG, int TS, int nblocks, const void *w,
                                  void *wf, size_t ws_bytes, hipStream_t s)
{
    const int total = nblocks * NCG * TS * 64;
    if (size_t(total) * 16 > ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_fwd_bf16, dim3(std::min((total + 255) / 256, 1024)), dim3(256), 0, s,
                       (const u16 *)w, (uint4 *)wf, g, NCG, TS, total);
    return hipGetLastError();
}

hipError_t launch_fwd_ig_bf16(const Geom &g, const FwdBfPlan &p, const void *x, const void *w,
                              const void *bias, void *y, void *ws, int relu, hipStream_t s)
{
    const FwdBfVariant *v = pick_fwd_bf(p.NW, p.MB, p.TS, p.NCG, p.G * p.nblk);
    if (!v) return hipErrorInvalidValue;
    // the packed weights cover every 16-channel block a wave of the grid reads
    const int nbt_grid = (g.OC + 16 * p.NW - 1) / (16 * p.NW) * p.NW;
    const int total = nbt_grid * p.NCG * p.TS * 64;
    if (size_t(total) * 16 > p.ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_fwd_bf16, dim3(std::min((total + 255) / 256, 1024)), dim3(256), 0, s,
                       (const u16 *)w, (uint4 *)ws, g, p.NCG, p.TS, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    FwdBfArgs a{g, (const u16 *)x, (const uint4 *)ws, (const u16 *)bias, (u16 *)y, relu, p.G, p.WP, p.IS, p.NCG, p.nblk};
    dim3 grid((g.B + p.G - 1) / p.G, (g.OC + 16 * p.NW - 1) / (16 * p.NW));
    e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
