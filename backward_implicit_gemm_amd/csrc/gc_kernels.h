// gc_kernels.h -- launchers of the gfx950 kernels, called by the C ABI layer.
#pragma once

#include "gc_common.h"

namespace gc {

// Shape-generic implicit GEMM (igemm_generic.hip).
template <typename T>
hipError_t launch_fwd_generic(const Geom &g, const void *x, const void *w, const void *bias,
                              void *y, int relu, hipStream_t s);
template <typename T>
hipError_t launch_dgrad_generic(const Geom &g, const void *dy, const void *w, const void *ym,
                                void *dx, int relu, hipStream_t s);
template <typename T>
hipError_t launch_wgrad_generic(const Geom &g, const void *x, const void *dy, const void *ym,
                                float *part, int splits, int relu, hipStream_t s);
int wgrad_generic_splits(const Geom &g);

// Image-group kernels on fp32 MFMA for shapes the kernels below do not plan
// (dgrad_ig_f32.hip, wgrad_ig_f32.hip).  plan_* returns false when a shape
// does not fit them.
struct DgradIgPlan;
struct WgradIgPlan;
struct DgradBfPlan;
struct WgradBfPlan;
struct WgradRfPlan;
struct BwdFusedBfPlan;
struct BwdFusedF32Plan;
// d_input and wgrad run on fp32 MFMA for both storage types (T = float or
// bf16_t; bf16 is widened exactly while staging).
bool plan_dgrad_ig_f32(const Geom &g, DgradIgPlan &p);
template <typename T>
hipError_t launch_dgrad_ig(const Geom &g, const DgradIgPlan &p, const void *dy, const void *w,
                           const void *ym, void *dx, int relu, hipStream_t s);
bool plan_wgrad_ig_f32(const Geom &g, WgradIgPlan &p);
template <typename T>
hipError_t launch_wgrad_ig(const Geom &g, const WgradIgPlan &p, const void *x, const void *dy,
                           const void *ym, float *part, int relu, hipStream_t s);

// Forward kernels with loader and MFMA waves.
struct FwdWsPlan;
// packs w into the B-fragment order of the bf16 forward for `nblocks`
// 16-channel blocks (fwd_pack.hip)
hipError_t launch_pack_w_fwd_bf16(const Geom &g, int NCG, int TS, int nblocks, const void *w,
                                  void *wf, size_t ws_bytes, hipStream_t s);
// bf16 forward with loader and MFMA waves; plan_* returns false when a shape
// does not fit it
bool plan_fwd_ws_bf16(const Geom &g, FwdWsPlan &p);
hipError_t launch_fwd_ws_bf16(const Geom &g, const FwdWsPlan &p, const void *x, const void *w,
                              const void *bias, void *y, void *ws, int relu, hipStream_t s);
// Bias gradient db[oc] = sum over (b, oh, ow) of dz (bias_grad.hip): fp32
// partials per image chunk in `part`, then the fixed-order reduction.
size_t bias_grad_ws_bytes(const Geom &g);
template <typename T>
hipError_t launch_bias_grad(const Geom &g, const void *dy, const void *ym, void *db, float *part,
                            int relu, hipStream_t s);
// packs w into the B-fragment order of the fp32 forward's MFMA steps (see
// FwdF32Steps) for `nblocks` 16-channel blocks (fwd_pack.hip)
hipError_t launch_pack_w_fwd_f32(const Geom &g, int NCG, int CPP, int TS, int lo, int nblocks,
                                 const void *w, void *wf, size_t ws_bytes, hipStream_t s);
// fp32 forward with loader and MFMA waves
bool plan_fwd_ws_f32(const Geom &g, FwdWsPlan &p);
hipError_t launch_fwd_ws_f32(const Geom &g, const FwdWsPlan &p, const void *x, const void *w,
                             const void *bias, void *y, void *ws, int relu, hipStream_t s);
// LDS pitch of the forwards' channels-innermost x tile (fwd_pack.hip)
void pick_lds_pitch(const Geom &g, int G, int MB, int TS, int &WP_out, int &IS_out);
bool plan_dgrad_ig_bf16(const Geom &g, DgradBfPlan &p);
// fp32 d_input on fp32 MFMA, weights read in place (dgrad_rf_f32.hip); the
// plan struct is shared with the bf16 kernel, KS holding the 16-channel
// blocks, and needs no workspace.
bool plan_dgrad_rf_f32(const Geom &g, DgradBfPlan &p);
hipError_t launch_dgrad_rf_f32(const Geom &g, const DgradBfPlan &p, const void *dy, const void *w,
                               const void *ym, void *dx, int relu, hipStream_t s);
// fp32 wgrad with image-quad staging: partial tiles then the fixed-order
// reduction into dw (fp32 storage only)
bool plan_wgrad_rf_f32(const Geom &g, WgradRfPlan &p);
// the same with the bias gradient as one more column (x = 1) of the tiles
bool plan_wgrad_rf_f32_bias(const Geom &g, WgradRfPlan &p);
// db (the bias gradient) is written when the plan has the bias column
hipError_t launch_wgrad_rf_f32(const Geom &g, const WgradRfPlan &p, const void *x, const void *dy,
                               const void *ym, void *dw, void *db, void *ws, int relu,
                               hipStream_t s);
// bf16 backward (d_input + wgrad) in three or four launches: pre-passes, both
// main kernels in one grid (or one after the other), reduction.  Same results
// as the separate calls.
bool plan_bwd_fused_bf16(const Geom &g, BwdFusedBfPlan &p);
hipError_t launch_bwd_fused_bf16(const Geom &g, const BwdFusedBfPlan &p, const void *x,
                                 const void *w, const void *dy, const void *ym, void *dx, void *dw,
                                 void *ws, int relu, hipStream_t s);
// fp32 backward in two launches: the d_input and wgrad workgroups in one
// grid, then the reduction.  Same results as the separate calls.
bool plan_bwd_fused_f32(const Geom &g, BwdFusedF32Plan &p);
hipError_t launch_bwd_fused_f32(const Geom &g, const BwdFusedF32Plan &p, const void *x,
                                const void *w, const void *dy, const void *ym, void *dx, void *dw,
                                void *ws, int relu, hipStream_t s);
bool plan_wgrad_ig_bf16(const Geom &g, WgradBfPlan &p);
// the same with the bias gradient as one more column (x = 1) of the tiles
bool plan_wgrad_ig_bf16_bias(const Geom &g, WgradBfPlan &p);
// the same for one given tile width (64*JW columns)
bool plan_wgrad_bf16_tiles(const Geom &g, int JW, WgradBfPlan &p, int bias = 0);
// dz regrouping, the partial-tile kernel and the fixed-order reduction into dw
hipError_t launch_wgrad_ig_bf16(const Geom &g, const WgradBfPlan &p, const void *x, const void *dy,
                                const void *ym, void *dw, void *db, void *ws, int relu,
                                hipStream_t s);
hipError_t launch_dgrad_ig_bf16(const Geom &g, const DgradBfPlan &p, const void *dy, const void *w,
                                const void *ym, void *dx, void *ws, int relu, hipStream_t s);

// Fixed-order sum of split partials, then the store in the output type
// (wgrad_reduce.hip).
template <typename T>
hipError_t launch_wgrad_reduce(const float *part, void *dw, int splits, int n, hipStream_t s);
// The same over partial rows of NP columns: columns 0..N-1 of row oc go to
// dw[oc][...], column N to db[oc], the rest (padding) nowhere.
template <typename T>
hipError_t launch_wgrad_reduce_bias(const float *part, void *dw, void *db, int splits, int OC, int N,
                                    int NP, hipStream_t s);

}  // namespace gc
