// wgrad_rf_f32_dev.h -- device code of the fp32 wgrad kernel (see
// wgrad_rf_f32.hip): the kernel body, taking its workgroup index, and a
// __global__ wrapper, so that the fused backward (bwd_fused_f32.hip) can run
// the body inside its own launch.
#pragma once
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


template <int NBWV, bool RELU, bool BIAS>
__device__ __forceinline__ void wgrad_rf_f32_body(const WgradRfArgs &a, int bid)
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
    const int xcd = int(bid) % nx, slot = int(bid) / nx;
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
    const int oslot = zslot + 1;                    // with the bias column: a slot of ones

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
    // B slot of column block nb at step s: xrow[s] * xm[nb] + coloff[nb]; the
    // bias column's lane takes xm = 0 and the slot of ones, so its B is 1 for
    // every image without a select in the MFMA loop
    int coloff[NBWV], xm[NBWV];
#pragma unroll
    for (int nb = 0; nb < NBWV; ++nb) {
        const int col = col0 + (nsub * NBWV + nb) * 16 + (lane & 15);
        const bool ones = BIAS && col == g.K;
        xm[nb] = ones ? 0 : 1;
        coloff[nb] = ones ? oslot : 0;
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
            if (BIAS) {
                lds4w[oslot] = make_float4(1.f, 1.f, 1.f, 1.f);
                lds4w[p.bufsz + oslot] = make_float4(1.f, 1.f, 1.f, 1.f);
            }
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
                        bv[nb] = buf[(BIAS ? xrow[s] * xm[nb] : xrow[s]) + coloff[nb]];
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

template <int NBWV, bool RELU, bool BIAS>
__global__ void __launch_bounds__(1024) wgrad_rf_f32(WgradRfArgs a)
{
    wgrad_rf_f32_body<NBWV, RELU, BIAS>(a, blockIdx.x);
}

}  // namespace
}  // namespace gc
