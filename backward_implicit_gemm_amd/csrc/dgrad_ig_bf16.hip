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
// issued one block ahead of its use.  The fp32 dcol tile goes to LDS, column
// by column, and the chunk's input gradient is gathered from it:
//     dx[b][ic][ih][iw] = sum over the taps with oh*S+kh = ih, ow*S+kw = iw
//                         of dcol[(oh,ow,b)][(ic,kh,kw)]
// Because the image index is innermost in m, one 16-byte LDS read returns a
// tap for four images at once.  The sum is in fp32 in a fixed tap order and
// rounded to bf16 once.  dcol is double-buffered, so one barrier per chunk
// separates the MFMA writes from the gather reads.
#include "gc_kernels.h"
#include "ig_common.h"

namespace gc {
namespace {

typedef unsigned short u16;

// Packed weights, 16-byte units ((chunk*NBC + nbl)*KS + ks)*64 + lane: column
// n = nbl*16 + lane%16 of the chunk is (icl, kk) = (n / KK, n % KK), and the
// unit holds w[32*ks + 8*(lane/16) + i][chunk*CC + icl][kk] for i = 0..7, zero
// past OC, IC or the chunk's CC*KK columns.
__global__ void __launch_bounds__(256) pack_w_dgrad_bf16(const u16 *__restrict__ w,
                                                         uint4 *__restrict__ wp, Geom g, int CC,
                                                         int NBC, int KS, int total)
{
    for (int u = blockIdx.x * 256 + threadIdx.x; u < total; u += gridDim.x * 256) {
        const int lane = u & 63;
        int rest = u >> 6;
        const int ks = rest % KS;
        rest /= KS;
        const int nbl = rest % NBC;
        const int chunk = rest / NBC;
        const int n = nbl * 16 + (lane & 15);
        const int icl = n / g.KK, kk = n - icl * g.KK;
        const int ic = chunk * CC + icl;
        const bool ok = icl < CC && ic < g.IC;
        const int oc0 = ks * 32 + (lane >> 4) * 8;
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

template <int NW, int MB, int KS, int TAPS>
__global__ void __launch_bounds__(64 * NW) dgrad_ig_bf16(DgradBfArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    const Geom &g = a.g;
    const DgradBfPlan &p = a.p;
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = p.G;
    const int b0 = blockIdx.x * G;
    const int gimg = min(G, g.B - b0);
    const int c_begin = blockIdx.y * p.cpg;
    const int c_end = min(c_begin + p.cpg, p.nchunks);

    u16 *dz = reinterpret_cast<u16 *>(lds4);                                   // [MB*16][OCP]
    float *dcol = reinterpret_cast<float *>(reinterpret_cast<char *>(lds4) + p.dz_bytes);
    const int dcol_buf = p.NBC * 16 * p.RP;                                    // [2][NBC*16][RP]

    // Padding rows (images past the batch, rows past G*P) and channels past
    // OC must read as zero.
    for (int i = tid; i < p.dz_bytes / 16; i += NT) lds4[i] = make_uint4(0, 0, 0, 0);

    // Gather role: this thread owns input pixel q of the (channel, image
    // quad) planes r0, r0 + rpi, ...  Pixel (ih, iw) takes the taps
    // oh*S + kh = ih, ow*S + kw = iw; their dcol offsets are fixed.
    const int rpi = NT / g.HW;
    const bool gthr = tid < rpi * g.HW;
    const int q = gthr ? tid % g.HW : 0;
    const int r0 = gthr ? tid / g.HW : 0;
    int toff[TAPS];
    int ntap = 0;
    {
        const int ih = q / g.W, iw = q % g.W;
#pragma unroll
        for (int j = 0; j < TAPS; ++j) toff[j] = 0;
        for (int oh = 0; oh < g.OH; ++oh) {
            const int kh = ih - oh * g.S;
            if (kh < 0 || kh >= g.KH) continue;
            for (int ow = 0; ow < g.OW; ++ow) {
                const int kw = iw - ow * g.S;
                if (kw < 0 || kw >= g.KW) continue;
                const int off = (kh * g.KW + kw) * p.RP + (oh * g.OW + ow) * G;
#pragma unroll
                for (int j = 0; j < TAPS; ++j)
                    if (j == ntap) toff[j] = off;
                ++ntap;
            }
        }
    }
    __syncthreads();

    // dz rows m = p*G + img, columns oc
    {
        const int n = gimg * g.OC * g.P;
        const size_t base = size_t(b0) * g.OC * g.P;
        for (int e = tid; e < n; e += NT) {
            uint32_t img, rem, oc, pp;
            fdivmod(e, a.fd_ocp, img, rem);
            fdivmod(rem, g.fd_P, oc, pp);
            u16 v = a.dy[base + e];
            if (a.relu && !(bf_to_f(a.ym[base + e]) > 0.f)) v = 0;
            dz[(int(pp) * G + int(img)) * p.OCP + int(oc)] = v;
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

    // This wave's column blocks: nbl = wave, wave + NW, ... of every chunk.
    auto nbc_of = [&](int c) {
        const int cc = min(p.CC, g.IC - c * p.CC);
        return (cc * g.KK + 15) >> 4;
    };
    int nc = c_begin, nn = wave;               // next block to load
    auto skip = [&]() {
        while (nc < c_end && nn >= nbc_of(nc)) {
            ++nc;
            nn = wave;
        }
    };
    uint4 bnext[KS];
    auto load_b = [&]() {
        const uint4 *src = a.wp + (size_t(nc) * p.NBC + nn) * KS * 64 + lane;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bnext[ks] = src[ks * 64];
    };
    skip();
    if (nc < c_end) load_b();

    for (int c = c_begin; c < c_end; ++c) {
        float *dbuf = dcol + ((c - c_begin) & 1) * dcol_buf;
        const int nbc = nbc_of(c);
        for (int nbl = wave; nbl < nbc; nbl += NW) {
            uint4 b[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) b[ks] = bnext[ks];
            nn += NW;
            skip();
            if (nc < c_end) load_b();
            f32x4 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[mb][ks], __builtin_bit_cast(bf16x8, b[ks]), acc[mb], 0, 0, 0);
            // lane holds rows mb*16 + 4*(lane/16) + v of column nbl*16 + lane%16
            float *dst = dbuf + (nbl * 16 + (lane & 15)) * p.RP + (lane >> 4) * 4;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4 *>(dst + mb * 16) = acc[mb];
        }
        __syncthreads();

        // gather the chunk's input gradient, four images per LDS read
        if (gthr) {
            const int c0 = c * p.CC;
            const int cc = min(p.CC, g.IC - c0);
            const int nquad = (gimg + 3) >> 2;
            for (int pl = r0; pl < cc * nquad; pl += rpi) {
                const int quad = pl / cc, icl = pl - quad * cc;
                const float *src = dbuf + icl * g.KK * p.RP + quad * 4;
                f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < TAPS; ++j)
                    if (j < ntap) s += *reinterpret_cast<const f32x4 *>(src + toff[j]);
                const int img0 = quad * 4;
                u16 *out = a.dx + (size_t(b0 + img0) * g.IC + c0 + icl) * g.HW + q;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (img0 + i < gimg) out[size_t(i) * g.IC * g.HW] = from_f32<bf16_t>(s[i]);
            }
        }
    }
}

struct DgradBfVariant {
    int NW, MB, KS, TAPS;
    void (*fn)(DgradBfArgs);
};

#define DB_V(MB, KS, TAPS) {8, MB, KS, TAPS, dgrad_ig_bf16<8, MB, KS, TAPS>}
#define DB_TAPS(MB, KS) DB_V(MB, KS, 2), DB_V(MB, KS, 4), DB_V(MB, KS, 9)
#define DB_KS(MB) DB_TAPS(MB, 1), DB_TAPS(MB, 2), DB_TAPS(MB, 4)
const DgradBfVariant kDgradBfVariants[] = {DB_KS(1), DB_KS(2), DB_KS(3), DB_KS(4)};
#undef DB_KS
#undef DB_TAPS
#undef DB_V

const DgradBfVariant *pick_dgrad_bf(int NW, int MB, int KS, int TAPS)
{
    for (const auto &v : kDgradBfVariants)
        if (v.NW == NW && v.MB == MB && v.KS == KS && v.TAPS == TAPS) return &v;
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
        const int RP = MB * 16 + 4;
        const size_t dz_bytes = size_t(MB) * 16 * OCP * 2;
        const int ngroups = (g.B + G - 1) / G;
        for (int CC = 1; CC <= g.IC; ++CC) {
            const int NBC = (CC * g.KK + 15) / 16;
            const size_t lds = dz_bytes + 2 * size_t(NBC) * 16 * RP * 4;
            if (lds > 160 * 1024) break;
            const int nchunks = (g.IC + CC - 1) / CC;
            const int occ = lds <= 80 * 1024 ? 2 : 1;
            int cgroups = 1;
            while (ngroups * cgroups < 256 * occ && cgroups < nchunks) ++cgroups;
            const int cpg = (nchunks + cgroups - 1) / cgroups;
            cgroups = (nchunks + cpg - 1) / cpg;
            // cycles per chunk on one CU
            const double mfma = double((NBC + NW - 1) / NW) * MB * KS * 16 * (NW / 4);
            const double passes = double((CC * (G / 4) + rpi - 1) / rpi);
            const double gather = passes * NW * (mt * 8.0 + 16.0);
            const double chunk = mfma + gather + 400.0;
            const double per_wg = cpg * chunk + 2500.0;
            const double waves_of_wgs = std::ceil(double(ngroups) * cgroups / (256.0 * occ));
            const double t = waves_of_wgs * per_wg * (occ == 2 ? 1.4 : 1.0);
            if (t < best - 1e-9) {
                if (!pick_dgrad_bf(NW, MB, KS, TAPS)) continue;
                best = t;
                p.NW = NW; p.G = G; p.MB = MB; p.KS = KS; p.TAPS = TAPS;
                p.CC = CC; p.NBC = NBC; p.nchunks = nchunks; p.cgroups = cgroups; p.cpg = cpg;
                p.RP = RP; p.OCP = OCP; p.dz_bytes = int(dz_bytes);
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
    const DgradBfVariant *v = pick_dgrad_bf(p.NW, p.MB, p.KS, p.TAPS);
    if (!v || g.HW > 64 * p.NW || p.G % 4 || p.G * g.P > 16 * p.MB) return hipErrorInvalidValue;
    const int total = p.nchunks * p.NBC * p.KS * 64;
    if (size_t(total) * 16 > p.ws_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_w_dgrad_bf16, dim3(std::min((total + 255) / 256, 2048)), dim3(256), 0, s,
                       (const u16 *)w, (uint4 *)ws, g, p.CC, p.NBC, p.KS, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DgradBfArgs a{g, (const u16 *)dy, (const u16 *)ym, (const uint4 *)ws, (u16 *)dx, relu, p,
                  make_fastdiv(g.OC * g.P)};
    e = allow_max_lds(reinterpret_cast<const void *>(v->fn));
    if (e != hipSuccess) return e;
    dim3 grid((g.B + p.G - 1) / p.G, p.cgroups);
    hipLaunchKernelGGL(v->fn, grid, dim3(64 * p.NW), p.lds, s, a);
    return hipGetLastError();
}

}  // namespace gc
