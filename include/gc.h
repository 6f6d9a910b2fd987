/*
 * gc.h -- C ABI of libgc: 2-D convolution forward, d_input and wgrad as
 * im2col-free implicit GEMMs on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one benchmarked in "Speedups to gemm_conv_forward and
 * gemm_conv_backward kernels" (PufferLib pull request #522): a forward conv
 * with an optional fused ReLU (the relu=1/relu=0 flag of its layer-1 and
 * layer-2 benchmark lines), and a backward pass that produces the weight
 * gradient ("wgrad") and the input gradient ("d_input"), in fp32 or bf16
 * (its precision=fp32 / precision=bf16 runs).  Stride S, no padding, dilation
 * 1, one group.  Output size: OH = (H-KH)/S + 1, OW = (W-KW)/S + 1 (integer
 * division; the page's layer 1 maps 11x15, K=5, S=3 to 3x4).  The same page
 * also times a separate bias-gradient kernel for these layers; the bias
 * entry points below add a per-channel bias to the forward pass and compute
 * its gradient.
 *
 *   y [b,oc,oh,ow] = f( sum_{ic,kh,kw} x[b,ic,oh*S+kh,ow*S+kw] * w[oc,ic,kh,kw] )
 *   dz             = relu ? dy * (y > 0) : dy          (derivative 0 at 0)
 *   dx [b,ic,ih,iw] = sum over (oc,oh,ow,kh,kw) with oh*S+kh = ih and
 *                     ow*S+kw = iw of dz[b,oc,oh,ow] * w[oc,ic,kh,kw]
 *   dw [oc,ic,kh,kw] = sum_{b,oh,ow} dz[b,oc,oh,ow] * x[b,ic,oh*S+kh,ow*S+kw]
 *
 * Layouts: x, dx NCHW [B][IC][H][W]; w, dw OIHW [OC][IC][KH][KW]; y, dy NCHW
 * [B][OC][OH][OW]; all dense and contiguous.  Storage type GC_F32 (IEEE fp32)
 * or GC_BF16 (bfloat16, 16-bit words); every tensor of a call has that type.
 * Products are accumulated in fp32; bf16 outputs are rounded to nearest even.
 *
 * Conventions common to every entry point:
 *   - Pointers are device pointers (HBM), owned by the caller, at least
 *     4-byte aligned for fp32 and 2-byte aligned for bf16.  The library
 *     never allocates, frees or synchronises; it enqueues kernels on
 *     `stream` (a hipStream_t; NULL means the default stream) and returns.
 *   - Outputs are overwritten, never accumulated into; every element is
 *     written, including exact zeros (input pixels no window covers).
 *   - Scratch memory, where an operation needs it, is passed in as
 *     `workspace` of `ws_bytes` bytes (device memory, 256-byte aligned);
 *     gc_conv_workspace_bytes() gives the size.  NULL/0 is fine when that
 *     size is 0.  Calls that overlap in time must not share a workspace.
 *   - Errors: an invalid descriptor, flag, dtype or a NULL pointer returns
 *     GC_ERR_INVALID_ARG before any HIP call; a workspace that is too small
 *     returns GC_ERR_WORKSPACE; shapes the kernels cannot tile return
 *     GC_ERR_UNSUPPORTED; a failed launch returns GC_ERR_HIP.  Nothing is
 *     enqueued when an error is returned before the launch.
 *   - Every element count (B*IC*H*W, B*OC*OH*OW, OC*IC*KH*KW) must be below
 *     2^31; larger tensors are rejected with GC_ERR_INVALID_ARG.
 *   - Entry points are reentrant.  The only state is an internal,
 *     thread-safe cache of kernel plans per problem shape.
 */
#ifndef GC_H
#define GC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GC_OK = 0,
    GC_ERR_INVALID_ARG = 1,
    GC_ERR_UNSUPPORTED = 2,
    GC_ERR_WORKSPACE = 3,
    GC_ERR_HIP = 4
} gc_status;

typedef enum { GC_F32 = 0, GC_BF16 = 1 } gc_dtype;

typedef enum {
    GC_OP_FWD = 0,          /* gc_conv_fwd and gc_conv_fwd_bias */
    GC_OP_BWD_DATA = 1,     /* gc_conv_bwd_data */
    GC_OP_BWD_WEIGHT = 2,   /* gc_conv_bwd_weight */
    GC_OP_BWD_BIAS = 3,     /* gc_conv_bwd_bias */
    GC_OP_BWD = 4,          /* gc_conv_bwd */
    GC_OP_BWD_WEIGHT_BIAS = 5   /* gc_conv_bwd_weight_bias */
} gc_op;

/* Problem size.  No padding, dilation 1, one group. */
typedef struct {
    int B, IC, H, W;   /* input  [B][IC][H][W] */
    int OC, KH, KW;    /* weight [OC][IC][KH][KW] */
    int stride;        /* S >= 1, the same along h and w */
} gc_conv_desc;

/* Output extent (pure host arithmetic).  Returns GC_OK and sets *OH, *OW, or
 * GC_ERR_INVALID_ARG for a descriptor with any dimension < 1, H < KH, W < KW,
 * stride < 1, or an element count of 2^31 or more. */
int gc_conv_out_dims(const gc_conv_desc *d, int *OH, int *OW);

/* Bytes of workspace that operation `op` needs for this problem and dtype
 * (0 if none).  Returns 0 as well for an invalid descriptor. */
size_t gc_conv_workspace_bytes(int op, const gc_conv_desc *d, int dtype);

/* Forward pass: y = f(conv(x, w)), f = ReLU when relu == 1, identity when
 * relu == 0.  x [B][IC][H][W], w [OC][IC][KH][KW] in, y [B][OC][OH][OW] out. */
int gc_conv_fwd(const void *x, const void *w, void *y,
                void *workspace, size_t ws_bytes,
                const gc_conv_desc *d, int relu, int dtype, void *stream);

/* The forward pass of gc_conv_fwd, for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace, the same results bit
 * for bit.  Its scratch memory (the packed weights) is a static device array
 * of 2 MiB per GPU, held by each GPU the library runs on until the process
 * ends; it covers both layer shapes of the PR page at every batch size, and
 * a problem whose gc_conv_workspace_bytes(GC_OP_FWD, ...) exceeds it returns
 * GC_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU shares that
 * GPU's array, so calls that may overlap in time on one GPU (on different
 * streams, or from different threads) race and must not be issued; calls
 * on one stream are ordered and safe.  It never allocates or frees memory. */
int gc_conv_fwd_noalloc(const void *x, const void *w, void *y,
                        const gc_conv_desc *d, int relu, int dtype, void *stream);

/* Forward pass with a bias: y = f(conv(x, w) + bias[oc]).  bias [OC] has the
 * storage type and is added in fp32 before the ReLU; everything else is as in
 * gc_conv_fwd (same workspace size).  bias must not be NULL. */
int gc_conv_fwd_bias(const void *x, const void *w, const void *bias, void *y,
                     void *workspace, size_t ws_bytes,
                     const gc_conv_desc *d, int relu, int dtype, void *stream);

/* Bias gradient: db[oc] = sum_{b,oh,ow} dz[b,oc,oh,ow], dz = dy masked by
 * (y_mask > 0) when relu == 1 (y_mask NULL when relu == 0).  db [OC] out.
 * Summed in fp32 in two stages whose order is fixed by the shape (partials
 * per chunk of images in `workspace`, then an ordered sum), so the result is
 * bit-identical from run to run. */
int gc_conv_bwd_bias(const void *dy, const void *y_mask, void *db,
                     void *workspace, size_t ws_bytes,
                     const gc_conv_desc *d, int relu, int dtype, void *stream);

/* d_input: dx from dy and w.  With relu == 1, dy is masked by (y_mask > 0),
 * y_mask being the forward output y; y_mask must be NULL when relu == 0.
 * dy [B][OC][OH][OW], w [OC][IC][KH][KW], y_mask like dy; dx [B][IC][H][W]
 * out (gather form, no atomics: each dx element is written once). */
int gc_conv_bwd_data(const void *dy, const void *w, const void *y_mask, void *dx,
                     void *workspace, size_t ws_bytes,
                     const gc_conv_desc *d, int relu, int dtype, void *stream);

/* wgrad: dw from x and dy (masked by y_mask > 0 when relu == 1; y_mask NULL
 * when relu == 0).  The sum over B*OH*OW is split across workgroups into fp32
 * partials in `workspace` and finished by a fixed-order reduction, so the
 * result is bit-identical from run to run. */
int gc_conv_bwd_weight(const void *x, const void *dy, const void *y_mask, void *dw,
                       void *workspace, size_t ws_bytes,
                       const gc_conv_desc *d, int relu, int dtype, void *stream);

/* wgrad and the bias gradient together: dw as gc_conv_bwd_weight computes it
 * and db[oc] = sum_{b,oh,ow} dz[b,oc,oh,ow] as gc_conv_bwd_bias does (db [OC]
 * in the storage type; dz = dy masked by y_mask > 0 when relu == 1).  The PR
 * page times the bias gradient as a kernel of its own (its bias-grad lines);
 * here db is one more column of the wgrad tiles, whose x operand is 1, so
 * it is summed from the dz already staged for wgrad and finished by the same
 * fixed-order reduction (bit-identical from run to run).  Shapes whose wgrad
 * kernel has no such column run gc_conv_bwd_weight and gc_conv_bwd_bias.
 * Workspace: gc_conv_workspace_bytes(GC_OP_BWD_WEIGHT_BIAS, ...), 256-byte
 * aligned.  db must not be NULL. */
int gc_conv_bwd_weight_bias(const void *x, const void *dy, const void *y_mask, void *dw,
                            void *db, void *workspace, size_t ws_bytes,
                            const gc_conv_desc *d, int relu, int dtype, void *stream);

/* The whole backward of a layer in one call: dx as gc_conv_bwd_data and dw
 * as gc_conv_bwd_weight compute them, with the same arguments and the same
 * results bit for bit.  The PR page times d_input and wgrad together as one
 * "backward"; this entry point runs them with fewer launches: for bf16
 * shapes with a fused plan, one pre-pass launch (dz regrouping for wgrad and
 * weight packing for d_input), then the two main kernels -- in one launch
 * holding both grids side by side where the d_input grid fits the chip in
 * one round, else one after the other -- and the fixed-order reduction of
 * wgrad's partials; for fp32 shapes with a fused plan, one launch holding the
 * d_input and wgrad grids side by side, then the reduction; for other shapes
 * the two calls one after the other.  The workspace
 * (gc_conv_workspace_bytes(GC_OP_BWD, ...)) must be 256-byte aligned. */
int gc_conv_bwd(const void *x, const void *w, const void *dy, const void *y_mask, void *dx,
                void *dw, void *workspace, size_t ws_bytes,
                const gc_conv_desc *d, int relu, int dtype, void *stream);

/* Which kernels an operation would run for this problem (pure host; the
 * same selection the entry point makes, under the current kernel policy).
 * Writes a NUL-terminated description -- the kernel family and its tiling
 * parameters, e.g. "fwd_ws_bf16 G=4 NBW=2 ..." -- into buf (truncated to
 * buf_bytes - 1 characters).  op is a gc_op value.  Returns GC_OK, or
 * GC_ERR_INVALID_ARG for an invalid descriptor, op or dtype, a NULL buf or
 * buf_bytes == 0.  Enqueues nothing. */
int gc_conv_plan_name(int op, const gc_conv_desc *d, int dtype, char *buf, size_t buf_bytes);

/* Human-readable name of a status code. */
const char *gc_status_string(int status);

/* Index-mapper self-check (pure host): builds the magic-number divider for
 * `divisor` exactly as the kernels use it (Granlund & Montgomery, "Division
 * by invariant integers using multiplication", 1994), applies it to every
 * n in [0, n_end) with the same arithmetic the device performs, and returns
 * the number of quotients or remainders that differ from n / divisor and
 * n % divisor.  Requires 1 <= divisor and n_end <= 2^31; returns -1 otherwise. */
int64_t gc_fastdiv_selfcheck(uint32_t divisor, uint32_t n_end);

/* Kernel selection policy, process-wide.  GC_POLICY_AUTO (the default) runs
 * the image-group kernels wherever a shape fits them and the shape-generic
 * kernels elsewhere; GC_POLICY_GENERIC runs the shape-generic kernels for
 * every shape (used to test both families on the same problems).  Returns
 * the previous policy, or -1 for an unknown value (nothing changes).  Calls
 * already enqueued are not affected; set it only while no other thread is
 * issuing calls. */
enum { GC_POLICY_AUTO = 0, GC_POLICY_GENERIC = 1 };
int gc_set_kernel_policy(int policy);

/* Library version, as major*10000 + minor*100 + patch. */
int gc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GC_H */
