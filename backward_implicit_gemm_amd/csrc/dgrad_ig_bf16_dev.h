// dgrad_ig_bf16_dev.h -- device code of the bf16 d_input kernel (see
// dgrad_ig_bf16.hip): the weight-packing pre-pass and the kernel body, each
// as a body taking its workgroup index plus a __global__ wrapper, so that the
// fused backward (bwd_fused_bf16.hip) can run them inside its own launches.
#pragma once
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {


typedef unsigned short u16;

// Packed weights, 16-byte units ((chunk*NBC + nbl)*KS + ks)*64 + lane: column
// n = nbl*16 + lane%16 of the chunk is (icl, kk) = (n / KK, n % KK), and the
// unit holds w[32*ks + 8*(lane/16) + i][chunk*CC + icl][kk] for i = 0..7, zero
// past OC, IC or the chunk's CC*KK columns.
// Workgroup `bid` of `nblk` (256 threads each) packs units bid*256 + t,
// stepping by nblk*256; the unit index splits with divisors prepared on the
// host (fd_ks: KS, fd_nbc: NBC).
__device__ __forceinline__ void pack_w_dgrad_bf16_body(const u16 *__restrict__ w,
                                                       uint4 *__restrict__ wp, const Geom &g,
                                                       int CC, FastDiv fd_nbc, FastDiv fd_ks,
                                                       int total, int bid, int nblk)
{
    for (int u = bid * 256 + threadIdx.x; u < total; u += nblk * 256) {
        const int lane = u & 63;
        uint32_t rest, ks, chunk, nbl;
        fdivmod(uint32_t(u >> 6), fd_ks, rest, ks);
        fdivmod(rest, fd_nbc, chunk, nbl);
        const int n = int(nbl) * 16 + (lane & 15);
        uint32_t icl, kk;
        fdivmod(uint32_t(n), g.fd_KK, icl, kk);
        const int ic = int(chunk) * CC + int(icl);
        const bool ok = int(icl) < CC && ic < g.IC;
        const int oc0 = int(ks) * 32 + (lane >> 4) * 8;
        u16 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = (ok && oc0 + i < g.OC) ? w[(size_t(oc0 + i) * g.IC + ic) * g.KK + kk] : u16(0);
        uint4 o;
        o.x = v[0] | (uint32_t(v[1]) << 16);
        o.y = v[2] | (uint32_t(v[3]) << 16);
        o.z = v[4] | (uint32_t(v[5]) << 16);
        o.w = v[6] | (uint32_t(v[7]) << 16);
        wp[u] = o;
    }
}
__global__ void __launch_bounds__(256) __attribute__((unused)) pack_w_dgrad_bf16(const u16 *__restrict__ w,
                                                         uint4 *__restrict__ wp, Geom g, int CC,
                                                         FastDiv fd_nbc, FastDiv fd_ks, int total)
{
    pack_w_dgrad_bf16_body(w, wp, g, CC, fd_nbc, fd_ks, total, blockIdx.x, gridDim.x);
}

struct DgradBfArgs {
    Geom g;
    const u16 *dy, *ym;
    const uint4 *wp;
    u16 *dx;
    int relu;
    DgradBfPlan p;
    FastDiv fd_ocp;    // OC*P: dz elements per image
};

__device__ __forceinline__ float bf_to_f(u16 v) { return __uint_as_float(uint32_t(v) << 16); }

// 16 bytes from a 2-byte-aligned global address (one global_load_dwordx4).
__device__ __forceinline__ uint4 ldg16_any(const u16 *p)
{
    uint4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

__device__ __forceinline__ u16 half_of(const uint4 &v, int i)
{
    const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return u16((i & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// The kernel body for workgroup (bx, by) of the (image group, channel group) grid.
template <int NW, int MB, int KS, int TAPS, int NBW, int GP>
__device__ __forceinline__ void dgrad_ig_bf16_body(const DgradBfArgs &a, int bx, int by)
{
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    const DgradBfPlan &p = a.p;
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = p.G;
    const int b0 = bx * G;
    const int gimg = min(G, g.B - b0);
    const int c_begin = by * p.cpg;
    const int c_end = min(c_begin + p.cpg, p.nchunks);

    u16 *dz = reinterpret_cast<u16 *>(lds4);                                   // [MB*16][OCP]
    float *dcol = reinterpret_cast<float *>(reinterpret_cast<char *>(lds4) + p.dz_bytes);
    const int dcol_buf = p.NBC * 16 * p.RP;                                    // [2][NBC*16][RP]
    u16 *otile = reinterpret_cast<u16 *>(dcol + 2 * dcol_buf);                // [2][G][ORUN]
    const int obuf = G * p.ORUN;
    const int zrow = MB * 16;        // rows zrow .. zrow+G-1 of every dcol column stay zero

    // Zero the dz tile (padding rows and channels past OC must read as 0)
    // and the zero rows of dcol, which stand in for absent taps.
    for (int i = tid; i < p.dz_bytes / 16; i += NT) lds4[i] = make_uint4(0, 0, 0, 0);
    {
        const int per_col = G / 4, n = 2 * p.NBC * 16 * per_col;
        for (int i = tid; i < n; i += NT) {
            const int col = i / per_col, k = i - col * per_col;
            *reinterpret_cast<f32x4 *>(dcol + col * p.RP + zrow + 4 * k) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // The weight fragments of this wave's first chunk are requested now; each
    // later chunk's are requested one chunk ahead of their use.
    auto nbc_of = [&](int c) {
        const int cc = min(p.CC, g.IC - c * p.CC);
        return (cc * g.KK + 15) >> 4;
    };
    uint4 bcur[NBW][KS], bnext[NBW][KS];
    auto load_b = [&](int c, uint4 (&dst)[NBW][KS]) {
        const int nbc = nbc_of(c);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int nbl = min(wave + j * NW, nbc - 1);      // clamped: always a valid block
            const uint4 *src = a.wp + (uint32_t(c * p.NBC + nbl) * KS * 64 + lane);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) dst[j][ks] = src[ks * 64];
        }
    };
    if (c_begin < c_end) load_b(c_begin, bcur);

    // dz: the group's gimg*OC*P contiguous elements of dy (and y), 8 per
    // 16-byte load, all of a thread's loads in flight together; element
    // e = (img, oc, p) goes to LDS row m = p*G + img, column oc.  With a ReLU
    // the element is kept where y > 0: for bf16 bits, 0 < bits <= 0x7F80
    // (positive, finite or +inf; NaN and -0 excluded).
    __syncthreads();            // zero fill complete
    {
        const int n = gimg * g.OC * g.P;
        const int n8 = n >> 3;
        const uint32_t base = uint32_t(b0) * g.OC * g.P;
        const int step = G * p.OCP;
        // writes elements e0 .. e0+cnt-1 held in v/m (8 lanes of 16 bits)
        auto put8 = [&](int e0, const uint4 &v, const uint4 &m, int cnt) {
            uint32_t img, rem, oc, pp;
            fdivmod(uint32_t(e0), a.fd_ocp, img, rem);
            fdivmod(rem, g.fd_P, oc, pp);
            int dst = (int(pp) * G + int(img)) * p.OCP + int(oc);
            int ip = int(pp), ioc = int(oc);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i >= cnt) break;
                u16 x = half_of(v, i);
                if (a.relu && uint32_t(half_of(m, i)) - 1u >= 0x7F80u) x = 0;
                dz[dst] = x;
                // advance (img, oc, p) by one element in NCHW order
                ++ip;
                dst += step;
                if (ip == g.P) {
                    ip = 0;
                    ++ioc;
                    dst += 1 - g.P * step;
                    if (ioc == g.OC) {
                        ioc = 0;
                        dst += 1 * p.OCP - g.OC;   // next image: row + 1, column 0
                    }
                }
            }
        };
        constexpr int U = 4;
        uint4 dv[U], mv[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = tid + k * NT;
            dv[k] = mv[k] = make_uint4(0, 0, 0, 0);
            if (u < n8) {
                dv[k] = ldg16_any(a.dy + base + 8 * u);
                if (a.relu) mv[k] = ldg16_any(a.ym + base + 8 * u);
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = tid + k * NT;
            if (u < n8) put8(8 * u, dv[k], mv[k], 8);
        }
        for (int u = tid + U * NT; u < n8; u += NT) {
            const uint4 v = ldg16_any(a.dy + base + 8 * u);
            const uint4 m = a.relu ? ldg16_any(a.ym + base + 8 * u) : make_uint4(0, 0, 0, 0);
            put8(8 * u, v, m, 8);
        }
        if (tid == 0 && 8 * n8 < n) {
            // the last n % 8 elements
            u16 tv[8] = {0, 0, 0, 0, 0, 0, 0, 0}, tm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int e = 8 * n8; e < n; ++e) {
                tv[e - 8 * n8] = a.dy[base + e];
                tm[e - 8 * n8] = a.relu ? a.ym[base + e] : u16(0);
            }
            uint4 v, m;
            v.x = tv[0] | (uint32_t(tv[1]) << 16); v.y = tv[2] | (uint32_t(tv[3]) << 16);
            v.z = tv[4] | (uint32_t(tv[5]) << 16); v.w = tv[6] | (uint32_t(tv[7]) << 16);
            m.x = tm[0] | (uint32_t(tm[1]) << 16); m.y = tm[2] | (uint32_t(tm[3]) << 16);
            m.z = tm[4] | (uint32_t(tm[5]) << 16); m.w = tm[6] | (uint32_t(tm[7]) << 16);
            put8(8 * n8, v, m, n - 8 * n8);
        }
    }

    // Gather role: this thread owns input pixel q of the (image quad,
    // channel) planes r0, r0 + rpi, ...  Pixel (ih, iw) takes the taps
    // oh*S + kh = ih, ow*S + kw = iw, i.e. oh in [oh_lo, oh_hi] and ow in
    // [ow_lo, ow_hi]; their dcol offsets are fixed.  Unused tap slots point
    // at the zero rows, so every thread issues the same TAPS reads and adds.
    const int rpi = NT / g.HW;
    const bool gthr = tid < rpi * g.HW;
    const int q = gthr ? tid % g.HW : 0;
    const int r0 = gthr ? tid / g.HW : 0;
    int toff[TAPS];
    {
        uint32_t ih, iw;
        fdivmod(uint32_t(q), g.fd_W, ih, iw);
        auto lo = [&](int i, int k) { return i - k + 1 <= 0 ? 0 : int(fdiv(uint32_t(i - k + g.S), g.fd_S)); };
        const int oh_lo = lo(int(ih), g.KH), oh_hi = min(g.OH - 1, int(fdiv(ih, g.fd_S)));
        const int ow_lo = lo(int(iw), g.KW), ow_hi = min(g.OW - 1, int(fdiv(iw, g.fd_S)));
#pragma unroll
        for (int j = 0; j < TAPS; ++j) toff[j] = zrow;
        int j = 0;
        for (int oh = oh_lo; oh <= oh_hi; ++oh)
            for (int ow = ow_lo; ow <= ow_hi; ++ow, ++j) {
                const int off = ((int(ih) - oh * g.S) * g.KW + int(iw) - ow * g.S) * p.RP +
                                (oh * g.OW + ow) * G;
#pragma unroll
                for (int t = 0; t < TAPS; ++t)
                    if (t == j) toff[t] = off;
            }
    }
    __syncthreads();

    // A fragments of every row block and oc step, kept for the whole kernel
    bf16x8 af[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const u16 *row = dz + (mb * 16 + (lane & 15)) * p.OCP + (lane >> 4) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            af[mb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(row + ks * 32));
    }

    // The chunk's dx tile, staged in LDS as [img][icl*HW + q], leaves in
    // 16-byte stores: for each image the chunk's cc*HW elements are
    // contiguous in dx.
    auto store_tile = [&](int c, const u16 *tile) {
        const int c0 = c * p.CC;
        const int run = min(p.CC, g.IC - c0) * g.HW;
        const int nu = (run + 7) >> 3;
        for (int u = tid; u < gimg * nu; u += NT) {
            const int img = u / nu, e0 = (u - img * nu) * 8;
            u16 *dst = a.dx + ((uint32_t(b0 + img) * g.IC + uint32_t(c0)) * g.HW + e0);
            const u16 *src = tile + img * p.ORUN + e0;
            if (e0 + 8 <= run) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src);
                __builtin_memcpy(dst, &v, sizeof(v));
            } else {
                for (int i = 0; i < run - e0; ++i) dst[i] = src[i];
            }
        }
    };

    for (int c = c_begin; c < c_end; ++c) {
        const int cb = (c - c_begin) & 1;
        float *dbuf = dcol + cb * dcol_buf;
        const int nbc = nbc_of(c);
        if (c + 1 < c_end) load_b(c + 1, bnext);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int nbl = wave + j * NW;
            if (nbl >= nbc) break;
            f32x4 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[mb][ks], __builtin_bit_cast(bf16x8, bcur[j][ks]), acc[mb], 0, 0, 0);
            // lane holds rows mb*16 + 4*(lane/16) + v of column nbl*16 + lane%16
            float *dst = dbuf + (nbl * 16 + (lane & 15)) * p.RP + (lane >> 4) * 4;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4 *>(dst + mb * 16) = acc[mb];
        }
        __syncthreads();
        // next chunk's fragments: the loads were issued a whole MFMA phase
        // ago; retire them before this iteration's stores are issued
        wait_vm();
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) bcur[j][ks] = bnext[j][ks];

        // the previous chunk's dx tile (complete since the barrier)
        if (c > c_begin) store_tile(c - 1, otile + (cb ^ 1) * obuf);

        // gather the chunk's input gradient, four images per LDS read;
        // plane pl = quad*cc + icl, this thread's planes r0 + k*rpi for
        // k < GP, all LDS reads issued before the first sum
        if (gthr) {
            const int cc = min(p.CC, g.IC - c * p.CC);
            const int nplanes = cc * ((gimg + 3) >> 2);
            int quad[GP], icl[GP];
            {
                int qd = 0, ic = r0;
                while (ic >= cc) { ic -= cc; ++qd; }
#pragma unroll
                for (int k = 0; k < GP; ++k) {
                    quad[k] = qd;
                    icl[k] = ic;
                    ic += rpi;
                    while (ic >= cc) { ic -= cc; ++qd; }
                }
            }
            f32x4 v[GP][TAPS];
#pragma unroll
            for (int k = 0; k < GP; ++k) {
                // planes past the chunk read plane 0 (valid LDS) and are not stored
                const bool on = r0 + k * rpi < nplanes;
                const float *src = dbuf + (on ? icl[k] * g.KK * p.RP + quad[k] * 4 : 0);
#pragma unroll
                for (int j = 0; j < TAPS; ++j) v[k][j] = *reinterpret_cast<const f32x4 *>(src + toff[j]);
            }
            u16 *ot = otile + cb * obuf;
#pragma unroll
            for (int k = 0; k < GP; ++k) {
                if (r0 + k * rpi >= nplanes) break;
                f32x4 sum = v[k][0];
#pragma unroll
                for (int j = 1; j < TAPS; ++j) sum += v[k][j];
                const int img0 = quad[k] * 4;
                u16 *o = ot + img0 * p.ORUN + icl[k] * g.HW + q;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (img0 + i < gimg) o[i * p.ORUN] = from_f32<bf16_t>(sum[i]);
            }
        }
    }
    __syncthreads();
    if (c_end > c_begin) store_tile(c_end - 1, otile + ((c_end - 1 - c_begin) & 1) * obuf);
}

template <int NW, int MB, int KS, int TAPS, int NBW, int GP>
__global__ void __launch_bounds__(64 * NW) dgrad_ig_bf16(DgradBfArgs a)
{
    dgrad_ig_bf16_body<NW, MB, KS, TAPS, NBW, GP>(a, blockIdx.x, blockIdx.y);
}

}  // namespace
}  // namespace gc
