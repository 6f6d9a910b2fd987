// dgrad_rf_f32_dev.h -- device code of the fp32 d_input kernel (see
// dgrad_rf_f32.hip): the kernel body, taking its workgroup coordinates, and a
// __global__ wrapper, so that the fused backward (bwd_fused_f32.hip) can run
// the body inside its own launch.
#pragma once
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

struct DgradRfArgs {
    Geom g;
    const float *dy, *ym;
    const float *w;      // OIHW weights, read in place
    float *dx;
    int relu;
    DgradBfPlan p;
    FastDiv fd_ocp;    // OC*P: dz elements per image
};

// KS4 = OC/16 rounded up: 16-channel blocks, each 4 MFMA steps of 4 channels.
//
// Roles: waves 0-7 (two per SIMD) run the MFMAs of chunk c while waves 8-15
// gather chunk c-1 and store its dx, all between the same pair of barriers,
// so the gather's LDS and VALU work hides under the MFMAs.  The roles branch
// outside the chunk loop (each wave passes the same number of barriers), so
// each role's registers are live only in its own loop.
template <int MB, int KS4, int TAPS, int NBW, bool EXACT>
__device__ __forceinline__ void dgrad_rf_f32_body(const DgradRfArgs &a, int bx, int by)
{
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    const DgradBfPlan &p = a.p;
    constexpr int NT = 1024, NMW = 8, NGT = 512;  // threads, MFMA waves, gather threads
    static_assert(NBW == 1, "one column block per MFMA wave");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool mfma_role = wave < NMW;
    const int G = p.G;
    const int b0 = bx * G;
    const int gimg = min(G, g.B - b0);
    const int c_begin = by * p.cpg;
    const int c_end = min(c_begin + p.cpg, p.nchunks);

    constexpr int KS = 4 * KS4;      // MFMA steps over oc
    float *dz = reinterpret_cast<float *>(lds4);                               // [MB*16][OCP]
    float *dcol = reinterpret_cast<float *>(reinterpret_cast<char *>(lds4) + p.dz_bytes);
    const int dcol_buf = p.NBC * 16 * p.RP;                                    // [2][NBC*16][RP]
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

    // ---- MFMA role: weights ------------------------------------------------
    // MFMA wave w (w < NBC) owns column block w of every chunk: weight-matrix
    // columns kc = chunk*CC*KK + 16*w + lane%16 of w[oc][ic*KK + kk].  Its B
    // values for 16-channel block s are w[16*s + 4*q + j][kc], j = 0..3 (q =
    // lane/16), four 4-byte loads in which 16 lanes read 16 consecutive floats
    // of one row.  They run D blocks ahead of their MFMAs through a register
    // ring that crosses chunk boundaries; the first D are issued here, before
    // the dz staging.  Every load stays inside the tensor: the column is
    // clamped to K-1 (columns past a chunk's CC*KK only feed dcol columns the
    // gather never reads, and the loads for the chunk after the last are
    // never used), and with OC < 16*KS4 (EXACT false) the rows past OC take
    // an offset past the end of the tensor, which reads zeros.
    constexpr int D = KS4 < 4 ? KS4 : 4;
    static_assert(KS4 % D == 0, "the ring slot of block s is s % D in every chunk");
    const bool mfma_on = mfma_role && wave < p.NBC;
    const uint32_t K4 = uint32_t(g.K) * 4;
    const int ckk = p.CC * g.KK;                                         // columns per chunk
    const __amdgpu_buffer_rsrc_t wrs = tensor_rsrc(a.w, uint32_t(g.OC) * K4);
    const uint32_t w_q = uint32_t(4 * (lane >> 4)) * K4;                // row 4*q
    int w_col = c_begin * ckk + wave * 16 + (lane & 15);                 // kc of the current chunk
    auto chunk_vo = [&](int col) { return w_q + uint32_t(min(col, g.K - 1)) * 4; };
    auto load_blk = [&](uint32_t vo, int s) {
        float4 r;
        if constexpr (EXACT) {
            r.x = bload4s(wrs, vo, uint32_t(16 * s + 0) * K4);
            r.y = bload4s(wrs, vo, uint32_t(16 * s + 1) * K4);
            r.z = bload4s(wrs, vo, uint32_t(16 * s + 2) * K4);
            r.w = bload4s(wrs, vo, uint32_t(16 * s + 3) * K4);
        } else {
            const int row = 16 * s + 4 * (lane >> 4);
            auto at = [&](int j) { return row + j < g.OC ? vo + uint32_t(16 * s + j) * K4 : kOffNone; };
            r.x = bload4s(wrs, at(0), 0);
            r.y = bload4s(wrs, at(1), 0);
            r.z = bload4s(wrs, at(2), 0);
            r.w = bload4s(wrs, at(3), 0);
        }
        return r;
    };
    float4 ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) ring[i] = mfma_on ? load_blk(chunk_vo(w_col), i) : make_float4(0.f, 0.f, 0.f, 0.f);

    // dz: the group's gimg*OC*P contiguous elements of dy (and y), 4 per
    // 16-byte load, all of a thread's loads in flight together; element
    // e = (img, oc, p) goes to LDS row m = p*G + img, column oc.  With a ReLU
    // the element is kept where y > 0.
    __syncthreads();            // zero fill complete
    {
        const int n = gimg * g.OC * g.P;
        const int n4 = n >> 2;
        const uint32_t base = uint32_t(b0) * g.OC * g.P;
        const int step = G * p.OCP;
        auto put4 = [&](int e0, const float4 &v, const float4 &m, int cnt) {
            uint32_t img, rem, oc, pp;
            fdivmod(uint32_t(e0), a.fd_ocp, img, rem);
            fdivmod(rem, g.fd_P, oc, pp);
            int dst = (int(pp) * G + int(img)) * p.OCP + int(oc);
            int ip = int(pp), ioc = int(oc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= cnt) break;
                float x = comp(v, i);
                if (a.relu && !(comp(m, i) > 0.f)) x = 0.f;
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
        float4 dv[U], mv[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = tid + k * NT;
            dv[k] = mv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u < n4) {
                dv[k] = ld4_f32(a.dy + base + 4 * u);
                if (a.relu) mv[k] = ld4_f32(a.ym + base + 4 * u);
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = tid + k * NT;
            if (u < n4) put4(4 * u, dv[k], mv[k], 4);
        }
        for (int u = tid + U * NT; u < n4; u += NT) {
            const float4 v = ld4_f32(a.dy + base + 4 * u);
            const float4 m = a.relu ? ld4_f32(a.ym + base + 4 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
            put4(4 * u, v, m, 4);
        }
        if (tid == 0 && 4 * n4 < n) {
            float tv[4] = {0.f, 0.f, 0.f, 0.f}, tm[4] = {0.f, 0.f, 0.f, 0.f};
            for (int e = 4 * n4; e < n; ++e) {
                tv[e - 4 * n4] = a.dy[base + e];
                tm[e - 4 * n4] = a.relu ? a.ym[base + e] : 0.f;
            }
            put4(4 * n4, make_float4(tv[0], tv[1], tv[2], tv[3]),
                 make_float4(tm[0], tm[1], tm[2], tm[3]), n - 4 * n4);
        }
    }

    // Gather role (threads 256..511): thread gt owns input pixel q of the
    // (image quad, channel) planes r0, r0 + rpi, ...  Pixel (ih, iw) takes
    // the taps oh*S + kh = ih, ow*S + kw = iw, i.e. oh in [oh_lo, oh_hi] and
    // ow in [ow_lo, ow_hi]; their dcol offsets are fixed.  Unused tap slots
    // point at the zero rows, so every thread issues the same TAPS reads.
    const int gt = tid - NMW * 64;
    const int rpi = NGT / g.HW;
    const bool gthr = !mfma_role && gt < rpi * g.HW;
    const int q = gthr ? gt % g.HW : 0;
    const int r0 = gthr ? gt / g.HW : 0;
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

    // ---- pipeline: iteration it computes chunk it and gathers chunk it-1;
    // every dcol buffer changes hands at a barrier -----------------------------
    if (!mfma_role) {
        // Gather role: sum the taps of 4 images per 16-byte read and store
        // straight to dx; a store instruction covers 64 consecutive pixels of
        // one plane, so the 4-byte stores coalesce without staging.  A chunk's
        // (channel, image quad) planes are numbered pl = icl*nq + quad; thread
        // (r0, q) takes planes r0, r0 + rpi, ... (at most NPL), whose LDS and
        // dx offsets are the same in every chunk up to the dcol buffer and the
        // chunk's first channel.  Images past the batch have dx offsets past
        // the end of the tensor, so their stores are dropped.
        constexpr int NPL = 4;
        const uint32_t plane4 = uint32_t(g.IC) * g.HW * 4;          // dx bytes per image
        const __amdgpu_buffer_rsrc_t dxrs = tensor_rsrc(a.dx, uint32_t(g.B) * plane4);
        const int nq = (gimg + 3) >> 2;
        int loff[NPL];
        uint32_t goff[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int pl = r0 + k * rpi;
            const int icl = pl / nq, quad = pl - icl * nq;
            loff[k] = icl * g.KK * p.RP + quad * 4;
            goff[k] = ((uint32_t(b0 + 4 * quad) * g.IC + uint32_t(icl)) * g.HW + uint32_t(q)) * 4;
        }
        for (int it = c_begin; it <= c_end; ++it) {
            if (it > c_begin && gthr) {
                const int c0 = (it - 1) * p.CC;
                const int nplanes = min(p.CC, g.IC - c0) * nq;
                const float *dbuf = dcol + ((it - 1 - c_begin) & 1) * dcol_buf;
                const uint32_t cbase = uint32_t(c0) * g.HW * 4;
#pragma unroll
                for (int k = 0; k < NPL; ++k) {
                    if (r0 + k * rpi < nplanes) {
                        const float *src = dbuf + loff[k];
                        f32x4 v[TAPS];
#pragma unroll
                        for (int j = 0; j < TAPS; ++j) v[j] = *reinterpret_cast<const f32x4 *>(src + toff[j]);
                        f32x4 sum = v[0];
#pragma unroll
                        for (int j = 1; j < TAPS; ++j) sum += v[j];
#pragma unroll
                        for (int i = 0; i < 4; ++i) bstore4s(dxrs, sum[i], goff[k] + i * plane4, cbase);
                    }
                }
            }
            __syncthreads();
        }
        return;
    }
    if (!mfma_on) {             // no column block for this wave
        for (int it = c_begin; it <= c_end; ++it) __syncthreads();
        return;
    }
    // A values come from the dz tile in LDS one 16-channel block ahead of
    // their MFMAs: lane (row mb*16 + lane%16, group q) reads dz[row][16*s +
    // 4*q .. +3].  C: lane holds rows mb*16 + 4*(lane/16) + v of column
    // wave*16 + lane%16.
    const float *arow = dz + (lane & 15) * p.OCP + 4 * (lane >> 4);
    float *dst = dcol + (wave * 16 + (lane & 15)) * p.RP + (lane >> 4) * 4;
    for (int it = c_begin; it <= c_end; ++it) {
        if (it < c_end) {
            f32x4 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
            float4 av[2][MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                av[0][mb] = *reinterpret_cast<const float4 *>(arow + mb * 16 * p.OCP);
            const uint32_t vo = chunk_vo(w_col), vo_next = chunk_vo(w_col + ckk);
#pragma unroll
            for (int s = 0; s < KS4; ++s) {
                if (s + 1 < KS4) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        av[(s + 1) & 1][mb] =
                            *reinterpret_cast<const float4 *>(arow + mb * 16 * p.OCP + 16 * (s + 1));
                }
                const float4 bv = ring[s % D];
                // refill: block s+D of this chunk, else block s+D-KS4 of the next
                ring[s % D] = s + D < KS4 ? load_blk(vo, s + D) : load_blk(vo_next, s + D - KS4);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(av[s & 1][mb], j), comp(bv, j),
                                                                       acc[mb], 0, 0, 0);
                // keep each block's loads and MFMAs in their place
                __builtin_amdgcn_sched_barrier(0);
            }
            float *d = dst + ((it - c_begin) & 1) * dcol_buf;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4 *>(d + mb * 16) = acc[mb];
            w_col += ckk;
        }
        __syncthreads();
    }
}

template <int MB, int KS4, int TAPS, int NBW, bool EXACT>
__global__ void __launch_bounds__(1024) dgrad_rf_f32(DgradRfArgs a)
{
    dgrad_rf_f32_body<MB, KS4, TAPS, NBW, EXACT>(a, blockIdx.x, blockIdx.y);
}

}  // namespace
}  // namespace gc
