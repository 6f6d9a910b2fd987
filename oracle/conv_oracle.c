/*
 * conv_oracle.c -- CPU oracle for the 2-D convolution forward pass and its two
 * backward passes (d_input and wgrad), with an optional fused ReLU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * Source of the method: "Speedups to gemm_conv_forward and gemm_conv_backward
 * kernels" (PufferLib pull request #522).  Its benchmark output defines the
 * operation by its parameters: batch B, input channels IC, output channels OC,
 * an HxW input, a square KxK kernel at stride S with no padding, and a relu
 * flag (layer-1 and layer-2 correctness blocks); the backward pass yields the
 * weight gradient ("wgrad") and the input gradient ("d_input").  The implicit
 * GEMM on that page reaches exactly the convolution's definition up to the
 * order of summation, so this oracle is that definition written out as direct
 * loops, with every sum accumulated in fp64.  Readings of points the page
 * leaves open:
 *   - no padding, dilation 1, groups 1; the output size floors:
 *       OH = (H - KH) / S + 1,  OW = (W - KW) / S + 1
 *     (the page's layer-1 line maps 11x15, K=5, S=3 to 3x4, which needs the
 *     floor since (15-5)/3 is not an integer);
 *   - the kernel may be rectangular (KH != KW); the page only uses KH == KW;
 *   - ReLU: y = pre if pre > 0 else 0; its derivative is taken as 0 at 0, so
 *     the backward mask is (y_mask > 0) strictly, where y_mask is the forward
 *     output handed in by the caller (not recomputed here);
 *   - the plain passes have no bias; the *_bias functions add the bias
 *     forward and its gradient (see there).
 *
 * Layouts: x is NCHW [B][IC][H][W], w is OIHW [OC][IC][KH][KW], y/dy are NCHW
 * [B][OC][OH][OW].  All arrays are fp64.  OpenMP splits only over independent
 * output slices, so results do not depend on the thread count.
 */
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef long long i64;

/* Output extent along one axis: floor((in - k) / s) + 1, or -1 if invalid. */
int oracle_out_dim(int in, int k, int s)
{
    if (in < 1 || k < 1 || s < 1 || in < k) return -1;
    return (in - k) / s + 1;
}

/* Threads the parallel loops below will use. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static i64 idx4(i64 a, i64 A1, i64 b, i64 B1, i64 c, i64 C1, i64 d)
{
    return ((a * A1 + b) * B1 + c) * C1 + d;
}

/* The ReLU-masked output gradient at one output element. */
static double masked_dy(const double *dy, const double *y_mask, int relu, i64 i)
{
    if (relu && !(y_mask[i] > 0.0)) return 0.0;
    return dy[i];
}

/*
 * Forward: y[b,oc,oh,ow] = f( sum_{ic,kh,kw} x[b,ic,oh*S+kh,ow*S+kw] * w[oc,ic,kh,kw] ),
 * f = ReLU when relu != 0, identity otherwise.
 */
void oracle_conv_fwd(const double *x, const double *w, double *y,
                     int B, int IC, int H, int W, int OC, int KH, int KW,
                     int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (i64 b = 0; b < B; ++b)
        for (int oc = 0; oc < OC; ++oc)
            for (int oh = 0; oh < OH; ++oh)
                for (int ow = 0; ow < OW; ++ow) {
                    double acc = 0.0;
                    for (int ic = 0; ic < IC; ++ic)
                        for (int kh = 0; kh < KH; ++kh)
                            for (int kw = 0; kw < KW; ++kw)
                                acc += x[idx4(b, IC, ic, H, oh * S + kh, W, ow * S + kw)]
                                     * w[idx4(oc, IC, ic, KH, kh, KW, kw)];
                    if (relu && !(acc > 0.0)) acc = 0.0;
                    y[idx4(b, OC, oc, OH, oh, OW, ow)] = acc;
                }
}

/*
 * d_input, written as the adjoint of the forward pass: every use of
 * x[b,ic,oh*S+kh,ow*S+kw] in the forward sum contributes dz*w to its gradient,
 * with dz the ReLU-masked dy.  Input pixels that no output window covers end
 * at exactly 0.
 */
void oracle_conv_bwd_data(const double *dy, const double *w, const double *y_mask,
                          double *dx, int B, int IC, int H, int W, int OC,
                          int KH, int KW, int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (i64 b = 0; b < B; ++b) {
        double *dxb = dx + b * (i64)IC * H * W;
        for (i64 i = 0; i < (i64)IC * H * W; ++i) dxb[i] = 0.0;
        for (int oc = 0; oc < OC; ++oc)
            for (int oh = 0; oh < OH; ++oh)
                for (int ow = 0; ow < OW; ++ow) {
                    const double g = masked_dy(dy, y_mask, relu,
                                               idx4(b, OC, oc, OH, oh, OW, ow));
                    for (int ic = 0; ic < IC; ++ic)
                        for (int kh = 0; kh < KH; ++kh)
                            for (int kw = 0; kw < KW; ++kw)
                                dxb[((i64)ic * H + oh * S + kh) * W + ow * S + kw] +=
                                    g * w[idx4(oc, IC, ic, KH, kh, KW, kw)];
                }
    }
}

/* wgrad: dw[oc,ic,kh,kw] = sum_{b,oh,ow} dz[b,oc,oh,ow] * x[b,ic,oh*S+kh,ow*S+kw]. */
void oracle_conv_bwd_weight(const double *x, const double *dy, const double *y_mask,
                            double *dw, int B, int IC, int H, int W, int OC,
                            int KH, int KW, int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (i64 p = 0; p < (i64)OC * IC; ++p) {
        const int oc = (int)(p / IC), ic = (int)(p % IC);
        for (int kh = 0; kh < KH; ++kh)
            for (int kw = 0; kw < KW; ++kw) {
                double acc = 0.0;
                for (i64 b = 0; b < B; ++b)
                    for (int oh = 0; oh < OH; ++oh)
                        for (int ow = 0; ow < OW; ++ow)
                            acc += masked_dy(dy, y_mask, relu, idx4(b, OC, oc, OH, oh, OW, ow))
                                 * x[idx4(b, IC, ic, H, oh * S + kh, W, ow * S + kw)];
                dw[idx4(oc, IC, ic, KH, kh, KW, kw)] = acc;
            }
    }
}

/*
 * Bias.  The same page times a separate per-channel bias-gradient kernel for
 * these two layers at the encoder's batch (its bias-grad timing lines); the
 * layer then reads y = f(conv(x, w) + bias[oc]).  Forward with a bias, and
 * the bias gradient db[oc] = sum_{b,oh,ow} dz[b,oc,oh,ow] (dz the
 * ReLU-masked dy, as above).  d_input and wgrad do not change with a bias.
 */
void oracle_conv_fwd_bias(const double *x, const double *w, const double *bias, double *y,
                          int B, int IC, int H, int W, int OC, int KH, int KW,
                          int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (i64 b = 0; b < B; ++b)
        for (int oc = 0; oc < OC; ++oc)
            for (int oh = 0; oh < OH; ++oh)
                for (int ow = 0; ow < OW; ++ow) {
                    double acc = bias[oc];
                    for (int ic = 0; ic < IC; ++ic)
                        for (int kh = 0; kh < KH; ++kh)
                            for (int kw = 0; kw < KW; ++kw)
                                acc += x[idx4(b, IC, ic, H, oh * S + kh, W, ow * S + kw)]
                                     * w[idx4(oc, IC, ic, KH, kh, KW, kw)];
                    if (relu && !(acc > 0.0)) acc = 0.0;
                    y[idx4(b, OC, oc, OH, oh, OW, ow)] = acc;
                }
}

void oracle_conv_bwd_bias(const double *dy, const double *y_mask, double *db,
                          int B, int OC, int OH, int OW, int relu)
{
#pragma omp parallel for schedule(static)
    for (int oc = 0; oc < OC; ++oc) {
        double acc = 0.0;
        for (i64 b = 0; b < B; ++b)
            for (int oh = 0; oh < OH; ++oh)
                for (int ow = 0; ow < OW; ++ow)
                    acc += masked_dy(dy, y_mask, relu, idx4(b, OC, oc, OH, oh, OW, ow));
        db[oc] = acc;
    }
}

/*
 * Single-element forms, used to check sampled outputs at sizes where the
 * full passes take too long.  The d_input form here is the gather form: it
 * enumerates the taps (kh,kw) that map an output position onto input pixel
 * (ih,iw), i.e. (ih-kh) divisible by S with 0 <= (ih-kh)/S < OH, and the same
 * along w -- a different loop structure from the scatter form above.
 * `n` elements are evaluated; coordinates come as n-by-4 int arrays.
 */
void oracle_conv_fwd_at(const double *x, const double *w, const int *coords, int n,
                        double *out, int B, int IC, int H, int W, int OC,
                        int KH, int KW, int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    (void)B; (void)OC;
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (int s = 0; s < n; ++s) {
        const i64 b = coords[4 * s], oc = coords[4 * s + 1];
        const int oh = coords[4 * s + 2], ow = coords[4 * s + 3];
        double acc = 0.0;
        for (int ic = 0; ic < IC; ++ic)
            for (int kh = 0; kh < KH; ++kh)
                for (int kw = 0; kw < KW; ++kw)
                    acc += x[idx4(b, IC, ic, H, oh * S + kh, W, ow * S + kw)]
                         * w[idx4(oc, IC, ic, KH, kh, KW, kw)];
        if (relu && !(acc > 0.0)) acc = 0.0;
        out[s] = acc;
    }
}

void oracle_conv_bwd_data_at(const double *dy, const double *w, const double *y_mask,
                             const int *coords, int n, double *out,
                             int B, int IC, int H, int W, int OC,
                             int KH, int KW, int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    (void)B;
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (int s = 0; s < n; ++s) {
        const i64 b = coords[4 * s];
        const int ic = coords[4 * s + 1], ih = coords[4 * s + 2], iw = coords[4 * s + 3];
        double acc = 0.0;
        for (int kh = 0; kh < KH; ++kh) {
            const int th = ih - kh;
            if (th < 0 || th % S != 0 || th / S >= OH) continue;
            for (int kw = 0; kw < KW; ++kw) {
                const int tw = iw - kw;
                if (tw < 0 || tw % S != 0 || tw / S >= OW) continue;
                for (int oc = 0; oc < OC; ++oc)
                    acc += masked_dy(dy, y_mask, relu, idx4(b, OC, oc, OH, th / S, OW, tw / S))
                         * w[idx4(oc, IC, ic, KH, kh, KW, kw)];
            }
        }
        out[s] = acc;
    }
}

void oracle_conv_bwd_weight_at(const double *x, const double *dy, const double *y_mask,
                               const int *coords, int n, double *out,
                               int B, int IC, int H, int W, int OC,
                               int KH, int KW, int S, int relu)
{
    const int OH = oracle_out_dim(H, KH, S), OW = oracle_out_dim(W, KW, S);
    if (OH < 1 || OW < 1) return;
#pragma omp parallel for schedule(static)
    for (int s = 0; s < n; ++s) {
        const int oc = coords[4 * s], ic = coords[4 * s + 1];
        const int kh = coords[4 * s + 2], kw = coords[4 * s + 3];
        double acc = 0.0;
        for (i64 b = 0; b < B; ++b)
            for (int oh = 0; oh < OH; ++oh)
                for (int ow = 0; ow < OW; ++ow)
                    acc += masked_dy(dy, y_mask, relu, idx4(b, OC, oc, OH, oh, OW, ow))
                         * x[idx4(b, IC, ic, H, oh * S + kh, W, ow * S + kw)];
        out[s] = acc;
    }
}
