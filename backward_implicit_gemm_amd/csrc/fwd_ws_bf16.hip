// fwd_ws_bf16.hip -- forward convolution, bf16 storage, fp32 accumulation,
// with loader waves and MFMA waves.
//
// y = x * w as an implicit GEMM y[m][n] = sum_k A[m][k] * w[n][k], m =
// (b,oh,ow), n = oc, on v_mfma_f32_16x16x32_bf16, whose operands carry 8
// consecutive reduction elements per lane.  The reduction index is ordered
// (channel group of 8, tap, channel) so that both operands are single
// 16-byte reads: a workgroup owns G whole images, each channel group of them
// staged in LDS channels-innermost [group][image][pixel][8], so the A
// fragment of output row (b,oh,ow) and tap (kh,kw) is the 16 bytes at pixel
// (oh*S+kh, ow*S+kw) (the transposition from NCHW happens in registers, 8
// pixels x 8 channels per loader thread); the weights are packed per call into
// fragment order (fwd_pack.hip) and streamed from L2 through register rings.
// Channels are padded to a multiple of 8 and taps to a multiple of 4 with
// zero weights.
//
// Roles.  A wave's vector-memory counter is in
// order: when one wave issues both the x staging loads (from HBM) and the
// weight-ring loads (from L2), every ring wait after an x load also waits for
// that x load, and the MFMAs stall on HBM latency.  Here the two never share
// a wave:
//   * 4 loader waves issue the buffer loads of the whole x tile at once (one
//     register set per staging phase; channels past IC and images past the
//     batch use an offset past the end of x and read zeros; the last 8-pixel
//     block of a plane is moved back to end with it), then transpose and store
//     phase after phase, with a barrier after each;
//   * 4 MFMA waves (one per SIMD) each own NBW 16-channel blocks, stream their
//     weight fragments, and start on phase ph as soon as its barrier passes.
// With NBW = 2 each A fragment read from LDS feeds two MFMAs.  The whole x
// tile has its own LDS, so no phase waits for a buffer to drain.
//
// A workgroup walks image groups grp = blockIdx.x, + gridDim.x, ... (one per
// workgroup when the batch gives no more groups than the grid has slots).
// Only one workgroup fits on a CU (the x tile fills most of its LDS), so the
// next group is pipelined inside the workgroup instead: as soon as a loader
// thread has stored phase ph of the current group, it issues the loads of
// phase ph of its next group into the same registers, and stores them once
// the MFMA waves have finished phase ph of the current group (one barrier per
// phase, at least two phases per group).  The weight ring runs on from one
// group into the next without a break (its slot pattern repeats per group).
// Each MFMA wave writes a group's output through a private LDS region as
// contiguous 16-byte stores: scattered 2-byte stores would sit in its
// in-order memory counter ahead of the next group's ring loads.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

typedef unsigned short u16;

constexpr int kMfmaWaves = 4, kLoadWaves = 4;
constexpr int kThreads = 64 * (kMfmaWaves + kLoadWaves);
constexpr int kLoaders = 64 * kLoadWaves;

struct FwdWsArgs {
    Geom g;
    const u16 *x;
    const uint4 *wf;
    const u16 *bias;
    u16 *y;
    int relu;
    int G;        // images per workgroup
    int WP;       // LDS pixel slots per image row (>= W)
    int IS;       // LDS pixel slots per image (>= H*WP)
    int nblk;     // 8-pixel blocks per image plane
    int ystage;   // stage the output through LDS (every channel of every wave real, P*NBW*16 % 8 == 0)
    int ybase;    // 16-byte LDS slot where the waves' output staging regions start
};

template <int NBW, int MB, int TS, int NCG, int CPP, int D>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) fwd_ws_bf16(FwdWsArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    constexpr int NPH = (NCG + CPP - 1) / CPP;
    constexpr int NFRAG = NCG * TS;
    static_assert(NFRAG % D == 0, "the ring's slot pattern must repeat per image group");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ngroups = (g.B + a.G - 1) / a.G;
    const int nmine = (ngroups - int(blockIdx.x) + int(gridDim.x) - 1) / int(gridDim.x);
    const int gstride = a.G * a.IS;                  // 16-byte slots per channel group

    if (wave >= kMfmaWaves) {
        // ---- loader waves: unit (channel group, image, 8-pixel block) ----
        const int lt = tid - 64 * kMfmaWaves;
        const int units_per_cg = a.G * a.nblk;
        const int u_blk = lt % a.nblk, u_img = (lt / a.nblk) % a.G, u_cgl = lt / units_per_cg;
        const bool u_unit = u_cgl < CPP;
        const int u_w0 = min(8 * u_blk, g.HW - 8);
        const uint32_t plane = uint32_t(g.HW) * 2;
        const __amdgpu_buffer_rsrc_t xrs = tensor_rsrc(a.x, uint32_t(g.B) * g.IC * plane);
        uint32_t in[NPH][8][4];
        // loads of phase ph of image group grp (zeros past the batch)
        auto fetch = [&](int grp, int ph) {
            const int b0 = grp * a.G;
            const bool img_ok = u_img < min(a.G, g.B - b0);
            const uint32_t u_off = (uint32_t(b0 + u_img) * g.IC * g.HW + u_w0) * 2;
            const int cg = ph * CPP + u_cgl;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int ic = cg * 8 + c;
                const bool ok = u_unit && cg < NCG && img_ok && ic < g.IC;
                const uint4 v = bload16u(xrs, ok ? u_off + uint32_t(ic) * plane : kOffNone);
                in[ph][c][0] = v.x; in[ph][c][1] = v.y; in[ph][c][2] = v.z; in[ph][c][3] = v.w;
            }
        };
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) fetch(blockIdx.x, ph);
        const int ih0 = u_w0 / g.W, iw0 = u_w0 - ih0 * g.W;
        for (int i = 0; i < nmine; ++i) {
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            const int cg = ph * CPP + u_cgl;
            if (u_unit && cg < NCG) {
                // word j of pixel p = channels (2j, 2j+1) at pixel p
                uint4 *dst = lds4 + cg * gstride + u_img * a.IS;
                int ih = ih0, iw = iw0;
#pragma unroll
                for (int pp = 0; pp < 8; ++pp) {
                    const int wi = pp >> 1;
                    uint32_t o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo_src = in[ph][2 * j][wi], hi_src = in[ph][2 * j + 1][wi];
                        o[j] = (pp & 1) ? ((lo_src >> 16) | (hi_src & 0xFFFF0000u))
                                        : ((lo_src & 0xFFFFu) | (hi_src << 16));
                    }
                    dst[ih * a.WP + iw] = make_uint4(o[0], o[1], o[2], o[3]);
                    if (++iw == g.W) { iw = 0; ++ih; }
                }
            }
            // phase ph of the next group; the last group loads group 0 again
            // (in bounds, never stored) so that no branch guards the loads
            fetch(i + 1 < nmine ? int(blockIdx.x) + (i + 1) * int(gridDim.x) : 0, ph);
            __syncthreads();                         // phase ph is in LDS
        }
        }
        return;
    }

    // ---- MFMA waves: NBW 16-channel blocks each ----
    const int nb0 = (blockIdx.y * kMfmaWaves + wave) * NBW;
    // fragment f of block j streams through ring[j][f % D], D fragments
    // ahead: a buffer load at lane offset w_vo plus the constant (j*NFRAG +
    // f)*1024, so no per-fragment address is held in registers
    const __amdgpu_buffer_rsrc_t wrs = tensor_rsrc(a.wf, uint32_t(gridDim.y) * kMfmaWaves * NBW * NFRAG * 1024);
    const uint32_t w_vo = (uint32_t(nb0) * NFRAG * 64 + lane) * 16;
    uint4 ring[NBW][D];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < D; ++i) ring[j][i] = bload16us(wrs, w_vo, (j * NFRAG + i) * 1024);

    // rows past a group's images read image slots the loaders filled with
    // zeros (or nothing the epilogue stores)
    int rowoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = mb * 16 + (lane & 15);
        rowoff[mb] = 0;
        if (r < a.G * g.P) {
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

    for (int i = 0; i < nmine; ++i) {
    const int b0 = (int(blockIdx.x) + i * int(gridDim.x)) * a.G;
    const int rows = min(a.G, g.B - b0) * g.P;
    // The LDS read addresses are the same for every group; re-defining the
    // group stride opaquely in each iteration keeps the compiler from
    // computing all of them before the loop and holding them in registers.
    int gs = gstride;
    asm volatile("" : "+s"(gs));
    f32x4 acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[j][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        __syncthreads();                             // wait for phase ph
#pragma unroll
        for (int cg = ph * CPP; cg < (ph + 1) * CPP && cg < NCG; ++cg) {
            const uint4 *xb = lds4 + cg * gs;
            // A fragments one tap step ahead of their MFMAs (two register
            // sets), which leaves the registers for a deep weight ring
            uint4 af[2][MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) af[0][mb] = xb[rowoff[mb] + toff[0]];
#pragma unroll
            for (int st = 0; st < TS; ++st) {
                if (st + 1 < TS) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) af[(st + 1) & 1][mb] = xb[rowoff[mb] + toff[st + 1]];
                }
                const int f = cg * TS + st;
                bf16x8 bv[NBW];
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    bv[j] = __builtin_bit_cast(bf16x8, ring[j][f % D]);
                    // the fragment D ahead, into the next group's first ones
                    // (after the last group they are loaded and not used)
                    ring[j][f % D] = bload16us(wrs, w_vo, (j * NFRAG + (f + D) % NFRAG) * 1024);
                }
                // Without this the scheduler sinks each refill load down to
                // just before its use, D steps later, and waits for it there:
                // the ring would then hide no latency at all.
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, af[st & 1][mb]), bv[j], acc[j][mb], 0, 0, 0);
            }
        }
    }

    // epilogue: row r = mb*16 + 4*(lane/16) + v, column (nb0 + j)*16 + lane%16.
    // Staged: the wave's NBW*16 channels of each image are one contiguous run
    // of y (NBW*16*P elements), so they go through the wave's own LDS region
    // ([img][channel][position], bf16) and leave in 16-byte stores instead of
    // 2-byte ones.  Only this wave touches the region, and its LDS accesses
    // are in order, so no barrier is needed.
    if (a.ystage) {
        const int run = NBW * 16 * g.P;                          // elements per image
        u16 *st = reinterpret_cast<u16 *>(lds4 + a.ybase) + wave * a.G * run;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int nl = j * 16 + (lane & 15);
            const float bn = a.bias ? __uint_as_float(uint32_t(a.bias[nb0 * 16 + nl]) << 16) : 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = mb * 16 + (lane >> 4) * 4 + v;
                    if (r >= rows) continue;
                    uint32_t img, pp;
                    fdivmod(r, g.fd_P, img, pp);
                    float val = acc[j][mb][v] + bn;
                    if (a.relu && !(val > 0.f)) val = 0.f;
                    st[(int(img) * NBW * 16 + nl) * g.P + int(pp)] = from_f32<bf16_t>(val);
                }
        }
        __builtin_amdgcn_wave_barrier();
        const int units = run / 8, gimg = rows / g.P;
        for (int u = lane; u < gimg * units; u += 64) {
            const int img = u / units, k = u - img * units;
            const uint4 v = *reinterpret_cast<const uint4 *>(st + img * run + 8 * k);
            __builtin_memcpy(a.y + (size_t(b0 + img) * g.OC + nb0 * 16) * g.P + 8 * k, &v, 16);
        }
        __builtin_amdgcn_wave_barrier();     // the region is rewritten for the next group
        continue;
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int n = (nb0 + j) * 16 + (lane & 15);
        if (n >= g.OC) continue;
        const float bn = a.bias ? __uint_as_float(uint32_t(a.bias[n]) << 16) : 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = mb * 16 + (lane >> 4) * 4 + v;
                if (r >= rows) continue;
                uint32_t img, pp;
                fdivmod(r, g.fd_P, img, pp);
                float val = acc[j][mb][v] + bn;
                if (a.relu && !(val > 0.f)) val = 0.f;
                a.y[(size_t(b0 + int(img)) * g.OC + n) * g.P + int(pp)] = from_f32<bf16_t>(val);
            }
    }
    }
}

struct FwdWsVariant {
    int NBW, MB, TS, NCG, CPP;
    void (*fn)(FwdWsArgs);
};
#define WS_V(NBW, MB, TS, NCG, CPP, D) {NBW, MB, TS, NCG, CPP, fwd_ws_bf16<NBW, MB, TS, NCG, CPP, D>}
const FwdWsVariant kFwdWsVariants[] = {
    // 59 -> 128, 11x15, 5x5, stride 3 (12 rows per image)
    WS_V(2, 3, 7, 8, 3, 7),     // 4 images, 128 channels per workgroup
    WS_V(1, 3, 7, 8, 3, 14),    // 4 images, 64 channels (two column tiles)
    WS_V(2, 1, 7, 8, 8, 7),     // one image
    // 128 -> 128, 3x4, 3x3 (2 rows per image), 64 channels per workgroup
    WS_V(1, 1, 3, 16, 16, 16),  // up to 8 images
    WS_V(1, 2, 3, 16, 8, 16),   // 16 images
    WS_V(1, 4, 3, 16, 4, 16),   // 32 images
};
#undef WS_V

const FwdWsVariant *pick_fwd_ws(int NBW, int MB, int TS, int NCG, int CPP)
{
    for (const auto &v : kFwdWsVariants)
        if (v.NBW == NBW && v.MB == MB && v.TS == TS && v.NCG == NCG && v.CPP == CPP) return &v;
    return nullptr;
}

}  // namespace

// Enumerates the tilings that have an instantiation -- NBW 16-channel blocks
// per MFMA wave (2: 128 channels per workgroup, 1: 64 channels and twice the
// column tiles), G images per workgroup, MB = ceil(G*P/16) row blocks, CPP
// channel groups per staging phase for the 256 loader threads -- and keeps
// the one that (1) puts the most workgroups on the chip at once, up to one
// per CU, then (2) wastes the fewest MFMA rows, then (3) has the wider NBW
// (each A read feeds more MFMAs), then (4) the larger G (fewer passes of the
// weight stream per image).
bool plan_fwd_ws_bf16(const Geom &g, FwdWsPlan &p)
{
    if (g.P > 64 || g.KK > 36 || g.HW < 8) return false;
    if (size_t(g.B) * g.IC * g.HW * 2 >= (size_t(1) << 31)) return false;
    // the weight packing runs one grid row per 16-channel block (at most 65535)
    if ((g.OC + 15) / 16 > 65535) return false;
    const int TS = (g.KK + 3) / 4;
    const int NCG = (g.IC + 7) / 8;
    const int nblk = (g.HW + 7) / 8;
    bool found = false;
    int best_wgs = 0, best_nbw = 0, best_g = 0;
    double best_fill = 0.0;
    for (int NBW : {2, 1}) {
        const int ntile = (g.OC + 64 * NBW - 1) / (64 * NBW);
        for (int G = std::min(g.B, std::max(1, 64 / g.P)); G >= 1; --G) {
            FwdWsPlan q{};
            q.NBW = NBW; q.TS = TS; q.NCG = NCG; q.nblk = nblk; q.ntile = ntile; q.G = G;
            q.MB = (G * g.P + 15) / 16;
            const int units_per_cg = G * nblk;
            if (units_per_cg > kLoaders) continue;
            // as many channel groups per phase as the loaders can stage, or
            // fewer where only that has an instantiation
            q.CPP = std::min(NCG, kLoaders / units_per_cg);
            while (q.CPP >= 1 && !pick_fwd_ws(NBW, q.MB, TS, NCG, q.CPP)) --q.CPP;
            if (q.CPP < 1) continue;
            const long long groups = (g.B + G - 1) / G;
            const int wgs = int(std::min<long long>(groups * ntile, g.ncu));
            const double fill = double(G * g.P) / (16.0 * q.MB);
            const bool better =
                !found || wgs > best_wgs ||
                (wgs == best_wgs && (fill > best_fill + 1e-9 ||
                                     (fill > best_fill - 1e-9 &&
                                      (NBW > best_nbw || (NBW == best_nbw && G > best_g)))));
            if (!better) continue;
            pick_lds_pitch(g, G, q.MB, TS, q.WP, q.IS);
            q.lds = sizeof(uint4) * size_t(NCG) * G * q.IS;
            // output staging: one region per MFMA wave, G images x NBW*16
            // channels x P; used when y is 16-byte aligned (checked per call)
            q.ystage = g.OC % (64 * NBW) == 0 && (g.P * NBW * 16) % 8 == 0;
            if (q.ystage) q.lds += size_t(kMfmaWaves) * G * NBW * 16 * g.P * 2;
            if (q.lds > 150 * 1024) continue;
            q.ws_bytes = size_t(ntile) * kMfmaWaves * NBW * NCG * TS * 64 * 16;
            p = q;
            found = true;
            best_wgs = wgs; best_fill = fill; best_nbw = NBW; best_g = G;
        }
    }
    return found;
}

hipError_t launch_fwd_ws_bf16(const Geom &g, const FwdWsPlan &p, const void *x, const void *w,
                              const void *bias, void *y, void *ws, int relu, hipStream_t s)
{
    // every precondition is checked before the first launch
    const FwdWsVariant *v = pick_fwd_ws(p.NBW, p.MB, p.TS, p.NCG, p.CPP);
    if (!v || p.G * p.nblk * p.CPP > kLoaders || g.HW < 8 || p.G * g.P > 16 * p.MB)
        return hipErrorInvalidValue;
    if (p.ystage && g.OC % (64 * p.NBW)) return hipErrorInvalidValue;
    // 16-byte output stores need a 16-byte-aligned y (every run starts at a
    // multiple of 8 elements from it); any other y takes the 2-byte stores
    const int ystage = p.ystage && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    hipError_t e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    e = launch_pack_w_fwd_bf16(g, p.NCG, p.TS, p.ntile * kMfmaWaves * p.NBW, w, ws, p.ws_bytes, s);
    if (e != hipSuccess) return e;
    FwdWsArgs a{g, (const u16 *)x, (const uint4 *)ws, (const u16 *)bias, (u16 *)y, relu,
                p.G, p.WP, p.IS, p.nblk, ystage, p.NCG * p.G * p.IS};
    // one workgroup per CU (the x tile takes most of its LDS): at most one
    // round of workgroups, each walking its share of the image groups.  The
    // next group's phase ph overwrites this group's phase ph only two
    // barriers later if there are at least two phases; with one, every
    // workgroup takes a single group.
    const int ngroups = (g.B + p.G - 1) / p.G;
    const int nph = (p.NCG + p.CPP - 1) / p.CPP;
    const int gx = nph >= 2 ? std::min(ngroups, std::max(1, g.ncu / p.ntile)) : ngroups;
    hipLaunchKernelGGL(v->fn, dim3(gx, p.ntile), dim3(kThreads), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
