// gc_api.hip -- the C ABI declared in include/gc.h: argument validation, the
// output-size closed form, workspace sizing and kernel selection.  All
// validation happens before the first HIP call, so the error paths are
// testable on a machine without a GPU.
#include <limits.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "../../include/gc.h"
#include "gc_kernels.h"
#include "ig_common.h"

using namespace gc;

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool valid_dtype(int dtype) { return dtype == GC_F32 || dtype == GC_BF16; }

// Checks the descriptor and fills the geometry.  OH = (H-KH)/S + 1 and
// OW = (W-KW)/S + 1 with integer division (no padding; the floor drops the
// input rows/columns no window reaches).
int check_desc(const gc_conv_desc *d, Geom *g)
{
    if (!d) return GC_ERR_INVALID_ARG;
    if (d->B < 1 || d->IC < 1 || d->H < 1 || d->W < 1 || d->OC < 1 || d->KH < 1 ||
        d->KW < 1 || d->stride < 1)
        return GC_ERR_INVALID_ARG;
    if (d->H < d->KH || d->W < d->KW) return GC_ERR_INVALID_ARG;
    const long long OH = (d->H - d->KH) / d->stride + 1;
    const long long OW = (d->W - d->KW) / d->stride + 1;
    const long long nx = (long long)d->B * d->IC * d->H * d->W;
    const long long ny = (long long)d->B * d->OC * OH * OW;
    const long long nw = (long long)d->OC * d->IC * d->KH * d->KW;
    if (nx > INT_MAX || ny > INT_MAX || nw > INT_MAX) return GC_ERR_INVALID_ARG;
    if (g) *g = make_geom(d->B, d->IC, d->H, d->W, d->OC, d->KH, d->KW, d->stride);
    return GC_OK;
}

bool aligned(const void *p, int dtype)
{
    const uintptr_t a = dtype == GC_F32 ? 4 : 2;
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GC_OK : GC_ERR_HIP; }

std::atomic<int> g_policy{GC_POLICY_AUTO};

bool use_ig() { return g_policy.load(std::memory_order_relaxed) == GC_POLICY_AUTO; }

// Plans depend only on the geometry, and some take a search (the bf16
// forward's LDS pitch) that costs far more host time than a launch, so each
// planner's answers are kept per geometry, one table per planner (two
// planners may share a plan type).  Thread-safe; a full table overwrites its
// entries round-robin.
template <typename P, bool (*Planner)(const Geom &, P &)>
bool cached_plan(const Geom &g, P &out)
{
    struct Entry {
        int key[8];
        bool ok;
        P plan;
    };
    constexpr int kSlots = 64;
    static std::mutex m;
    static Entry table[kSlots];
    static int used = 0, next = 0;
    const int key[8] = {g.B, g.IC, g.H, g.W, g.OC, g.KH, g.KW, g.S};
    {
        std::lock_guard<std::mutex> lk(m);
        for (int i = 0; i < used; ++i)
            if (std::equal(key, key + 8, table[i].key)) {
                if (table[i].ok) out = table[i].plan;
                return table[i].ok;
            }
    }
    P p{};
    const bool ok = Planner(g, p);
    std::lock_guard<std::mutex> lk(m);
    Entry &e = table[used < kSlots ? used++ : (next++ % kSlots)];
    std::copy(key, key + 8, e.key);
    e.ok = ok;
    e.plan = p;
    if (ok) out = p;
    return ok;
}

bool fwd_f32_plan(const Geom &g, FwdIgPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_fwd_ig_f32>(g, p);
}
bool fwd_f32_rf_plan(const Geom &g, FwdBfPlan &p)
{
    return use_ig() && cached_plan<FwdBfPlan, plan_fwd_rf_f32>(g, p);
}
bool fwd_f32_ws_plan(const Geom &g, FwdWsPlan &p)
{
    return use_ig() && cached_plan<FwdWsPlan, plan_fwd_ws_f32>(g, p);
}
bool fwd_bf16_ws_plan(const Geom &g, FwdWsPlan &p)
{
    return use_ig() && cached_plan<FwdWsPlan, plan_fwd_ws_bf16>(g, p);
}
bool fwd_bf16_plan(const Geom &g, FwdBfPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_fwd_ig_bf16>(g, p);
}
bool dgrad_bf16_plan(const Geom &g, DgradBfPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_dgrad_ig_bf16>(g, p);
}
bool dgrad_f32_rf_plan(const Geom &g, DgradBfPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_dgrad_rf_f32>(g, p);
}
bool wgrad_bf16_plan(const Geom &g, WgradBfPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_wgrad_ig_bf16>(g, p);
}
bool dgrad_plan(const Geom &g, DgradIgPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_dgrad_ig_f32>(g, p);
}
bool bwd_fused_plan(const Geom &g, BwdFusedBfPlan &p)
{
    return use_ig() && cached_plan<BwdFusedBfPlan, plan_bwd_fused_bf16>(g, p);
}
size_t round256(size_t n) { return (n + 255) & ~size_t(255); }
bool wgrad_f32_rf_plan(const Geom &g, WgradRfPlan &p)
{
    return use_ig() && cached_plan<WgradRfPlan, plan_wgrad_rf_f32>(g, p);
}
bool wgrad_plan(const Geom &g, WgradIgPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_wgrad_ig_f32>(g, p);
}

// Number of fp32 partial tiles wgrad writes for this problem, and the plan
// of the image-group kernel when it runs.
int wgrad_splits(const Geom &g, int dtype, WgradIgPlan *ig, bool *use)
{
    WgradIgPlan p;
    if (wgrad_plan(g, p)) {
        if (ig) *ig = p;
        if (use) *use = true;
        return p.splits;
    }
    if (use) *use = false;
    return wgrad_generic_splits(g);
}

size_t wgrad_ws_bytes(const Geom &g, int dtype)
{
    WgradBfPlan bp;
    if (dtype == GC_BF16 && wgrad_bf16_plan(g, bp)) return bp.ws_bytes;
    WgradRfPlan rp;
    if (dtype == GC_F32 && wgrad_f32_rf_plan(g, rp)) return rp.ws_bytes;
    return size_t(wgrad_splits(g, dtype, nullptr, nullptr)) * g.OC * g.K * sizeof(float);
}

}  // namespace

extern "C" {

int gc_version(void) { return kVersion; }

const char *gc_status_string(int status)
{
    switch (status) {
    case GC_OK: return "GC_OK";
    case GC_ERR_INVALID_ARG: return "GC_ERR_INVALID_ARG: invalid descriptor, flag, dtype or pointer";
    case GC_ERR_UNSUPPORTED: return "GC_ERR_UNSUPPORTED: shape not supported by the kernels";
    case GC_ERR_WORKSPACE: return "GC_ERR_WORKSPACE: workspace missing or too small";
    case GC_ERR_HIP: return "GC_ERR_HIP: kernel launch failed";
    default: return "unknown gc status";
    }
}

int gc_conv_out_dims(const gc_conv_desc *d, int *OH, int *OW)
{
    Geom g;
    const int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (OH) *OH = g.OH;
    if (OW) *OW = g.OW;
    return GC_OK;
}

size_t gc_conv_workspace_bytes(int op, const gc_conv_desc *d, int dtype)
{
    Geom g;
    if (check_desc(d, &g) != GC_OK || !valid_dtype(dtype)) return 0;
    switch (op) {
    case GC_OP_FWD: {
        FwdWsPlan wp;
        if (dtype == GC_BF16 && fwd_bf16_ws_plan(g, wp)) return wp.ws_bytes;
        if (dtype == GC_F32 && fwd_f32_ws_plan(g, wp)) return wp.ws_bytes;
        FwdBfPlan p;
        if (dtype == GC_BF16 && fwd_bf16_plan(g, p)) return p.ws_bytes;
        if (dtype == GC_F32 && fwd_f32_rf_plan(g, p)) return p.ws_bytes;
        return 0;
    }
    case GC_OP_BWD_DATA: {
        DgradBfPlan p;
        if (dtype == GC_BF16 && dgrad_bf16_plan(g, p)) return p.ws_bytes;
        if (dtype == GC_F32 && dgrad_f32_rf_plan(g, p)) return p.ws_bytes;
        return 0;
    }
    case GC_OP_BWD_WEIGHT: return wgrad_ws_bytes(g, dtype);
    case GC_OP_BWD_BIAS: return bias_grad_ws_bytes(g);
    case GC_OP_BWD: {
        BwdFusedBfPlan p;
        if (dtype == GC_BF16 && bwd_fused_plan(g, p)) return p.ws_bytes;
        // d_input's workspace, then wgrad's at the next 256-byte boundary
        return round256(gc_conv_workspace_bytes(GC_OP_BWD_DATA, d, dtype)) +
               gc_conv_workspace_bytes(GC_OP_BWD_WEIGHT, d, dtype);
    }
    default: return 0;
    }
}

static int conv_fwd(const void *x, const void *w, const void *bias, void *y, void *workspace,
             size_t ws_bytes, const gc_conv_desc *d, int relu, int dtype, void *stream)
{
    Geom g;
    int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!x || !w || !y) return GC_ERR_INVALID_ARG;
    if (!aligned(x, dtype) || !aligned(w, dtype) || !aligned(y, dtype) ||
        (bias && !aligned(bias, dtype)))
        return GC_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == GC_F32) {
        FwdWsPlan wp;
        if (fwd_f32_ws_plan(g, wp)) {
            if (!workspace || ws_bytes < wp.ws_bytes) return GC_ERR_WORKSPACE;
            if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
            return hip_status(launch_fwd_ws_f32(g, wp, x, w, bias, y, workspace, relu, s));
        }
        FwdBfPlan rp;
        if (fwd_f32_rf_plan(g, rp)) {
            if (!workspace || ws_bytes < rp.ws_bytes) return GC_ERR_WORKSPACE;
            if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
            return hip_status(launch_fwd_rf_f32(g, rp, x, w, bias, y, workspace, relu, s));
        }
        FwdIgPlan p;
        if (fwd_f32_plan(g, p))
            return hip_status(launch_fwd_ig_f32(g, p, x, w, bias, y, relu, s));
        return hip_status(launch_fwd_generic<float>(g, x, w, bias, y, relu, s));
    }
    FwdWsPlan wp;
    if (fwd_bf16_ws_plan(g, wp)) {
        if (!workspace || ws_bytes < wp.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
        return hip_status(launch_fwd_ws_bf16(g, wp, x, w, bias, y, workspace, relu, s));
    }
    FwdBfPlan p;
    if (fwd_bf16_plan(g, p)) {
        if (!workspace || ws_bytes < p.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
        return hip_status(launch_fwd_ig_bf16(g, p, x, w, bias, y, workspace, relu, s));
    }
    return hip_status(launch_fwd_generic<bf16_t>(g, x, w, bias, y, relu, s));
}

int gc_conv_fwd(const void *x, const void *w, void *y, void *workspace, size_t ws_bytes,
                const gc_conv_desc *d, int relu, int dtype, void *stream)
{
    return conv_fwd(x, w, nullptr, y, workspace, ws_bytes, d, relu, dtype, stream);
}

int gc_conv_fwd_bias(const void *x, const void *w, const void *bias, void *y, void *workspace,
                     size_t ws_bytes, const gc_conv_desc *d, int relu, int dtype, void *stream)
{
    if (!bias) return GC_ERR_INVALID_ARG;
    return conv_fwd(x, w, bias, y, workspace, ws_bytes, d, relu, dtype, stream);
}

int gc_conv_bwd_bias(const void *dy, const void *y_mask, void *db, void *workspace,
                     size_t ws_bytes, const gc_conv_desc *d, int relu, int dtype, void *stream)
{
    Geom g;
    int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!dy || !db) return GC_ERR_INVALID_ARG;
    if ((relu == 1) != (y_mask != nullptr)) return GC_ERR_INVALID_ARG;
    if (!aligned(dy, dtype) || !aligned(db, dtype) || (y_mask && !aligned(y_mask, dtype)))
        return GC_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < bias_grad_ws_bytes(g)) return GC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *part = static_cast<float *>(workspace);
    return hip_status(dtype == GC_F32 ? launch_bias_grad<float>(g, dy, y_mask, db, part, relu, s)
                                      : launch_bias_grad<bf16_t>(g, dy, y_mask, db, part, relu, s));
}

int gc_conv_bwd_data(const void *dy, const void *w, const void *y_mask, void *dx,
                     void *workspace, size_t ws_bytes, const gc_conv_desc *d, int relu,
                     int dtype, void *stream)
{
    Geom g;
    int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!dy || !w || !dx) return GC_ERR_INVALID_ARG;
    if ((relu == 1) != (y_mask != nullptr)) return GC_ERR_INVALID_ARG;
    if (!aligned(dy, dtype) || !aligned(w, dtype) || !aligned(dx, dtype) ||
        (y_mask && !aligned(y_mask, dtype)))
        return GC_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        DgradBfPlan bp;
        const bool bf = dtype == GC_BF16 && dgrad_bf16_plan(g, bp);
        const bool rf = !bf && dtype == GC_F32 && dgrad_f32_rf_plan(g, bp);
        if (bf) {
            if (!workspace || ws_bytes < bp.ws_bytes) return GC_ERR_WORKSPACE;
            if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
            return hip_status(launch_dgrad_ig_bf16(g, bp, dy, w, y_mask, dx, workspace, relu, s));
        }
        if (rf) return hip_status(launch_dgrad_rf_f32(g, bp, dy, w, y_mask, dx, relu, s));
    }
    DgradIgPlan p;
    const bool ig = dgrad_plan(g, p);
    if (dtype == GC_F32)
        return hip_status(ig ? launch_dgrad_ig<float>(g, p, dy, w, y_mask, dx, relu, s)
                             : launch_dgrad_generic<float>(g, dy, w, y_mask, dx, relu, s));
    return hip_status(ig ? launch_dgrad_ig<bf16_t>(g, p, dy, w, y_mask, dx, relu, s)
                         : launch_dgrad_generic<bf16_t>(g, dy, w, y_mask, dx, relu, s));
}

int gc_conv_bwd_weight(const void *x, const void *dy, const void *y_mask, void *dw,
                       void *workspace, size_t ws_bytes, const gc_conv_desc *d, int relu,
                       int dtype, void *stream)
{
    Geom g;
    int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!x || !dy || !dw) return GC_ERR_INVALID_ARG;
    if ((relu == 1) != (y_mask != nullptr)) return GC_ERR_INVALID_ARG;
    if (!aligned(x, dtype) || !aligned(dy, dtype) || !aligned(dw, dtype) ||
        (y_mask && !aligned(y_mask, dtype)))
        return GC_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == GC_BF16) {
        WgradBfPlan bp;
        if (wgrad_bf16_plan(g, bp)) {
            if (!workspace || ws_bytes < bp.ws_bytes) return GC_ERR_WORKSPACE;
            if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
            return hip_status(launch_wgrad_ig_bf16(g, bp, x, dy, y_mask, dw, workspace, relu, s));
        }
    }
    if (dtype == GC_F32) {
        WgradRfPlan rp;
        if (wgrad_f32_rf_plan(g, rp)) {
            if (!workspace || ws_bytes < rp.ws_bytes) return GC_ERR_WORKSPACE;
            if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
            return hip_status(launch_wgrad_rf_f32(g, rp, x, dy, y_mask, dw, workspace, relu, s));
        }
    }
    WgradIgPlan ig;
    bool use_ig_path = false;
    const int splits = wgrad_splits(g, dtype, &ig, &use_ig_path);
    const size_t need = size_t(splits) * g.OC * g.K * sizeof(float);
    if (need && (!workspace || ws_bytes < need)) return GC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
    float *part = static_cast<float *>(workspace);
    hipError_t e;
    if (dtype == GC_F32) {
        if (use_ig_path)
            e = launch_wgrad_ig<float>(g, ig, x, dy, y_mask, part, relu, s);
        else
            e = launch_wgrad_generic<float>(g, x, dy, y_mask, part, splits, relu, s);
        if (e == hipSuccess) e = launch_wgrad_reduce<float>(part, dw, splits, g.OC * g.K, s);
    } else {
        if (use_ig_path)
            e = launch_wgrad_ig<bf16_t>(g, ig, x, dy, y_mask, part, relu, s);
        else
            e = launch_wgrad_generic<bf16_t>(g, x, dy, y_mask, part, splits, relu, s);
        if (e == hipSuccess) e = launch_wgrad_reduce<bf16_t>(part, dw, splits, g.OC * g.K, s);
    }
    return hip_status(e);
}

int gc_conv_bwd(const void *x, const void *w, const void *dy, const void *y_mask, void *dx,
                void *dw, void *workspace, size_t ws_bytes, const gc_conv_desc *d, int relu,
                int dtype, void *stream)
{
    Geom g;
    int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!x || !w || !dy || !dx || !dw) return GC_ERR_INVALID_ARG;
    if ((relu == 1) != (y_mask != nullptr)) return GC_ERR_INVALID_ARG;
    if (!aligned(x, dtype) || !aligned(w, dtype) || !aligned(dy, dtype) || !aligned(dx, dtype) ||
        !aligned(dw, dtype) || (y_mask && !aligned(y_mask, dtype)))
        return GC_ERR_INVALID_ARG;
    BwdFusedBfPlan fp;
    if (dtype == GC_BF16 && bwd_fused_plan(g, fp)) {
        if (!workspace || ws_bytes < fp.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
        return hip_status(launch_bwd_fused_bf16(g, fp, x, w, dy, y_mask, dx, dw, workspace, relu,
                                                static_cast<hipStream_t>(stream)));
    }
    // no fused plan: d_input, then wgrad, each in its part of the workspace
    const size_t wd = gc_conv_workspace_bytes(GC_OP_BWD_DATA, d, dtype);
    const size_t ww = gc_conv_workspace_bytes(GC_OP_BWD_WEIGHT, d, dtype);
    const size_t off = round256(wd);
    if (off + ww > 0 && (!workspace || ws_bytes < off + ww)) return GC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
    st = gc_conv_bwd_data(dy, w, y_mask, dx, wd ? workspace : nullptr, wd, d, relu, dtype, stream);
    if (st != GC_OK) return st;
    void *wsw = ww ? static_cast<char *>(workspace) + off : nullptr;
    return gc_conv_bwd_weight(x, dy, y_mask, dw, wsw, ww, d, relu, dtype, stream);
}

int gc_set_kernel_policy(int policy)
{
    if (policy != GC_POLICY_AUTO && policy != GC_POLICY_GENERIC) return -1;
    return g_policy.exchange(policy);
}

int64_t gc_fastdiv_selfcheck(uint32_t divisor, uint32_t n_end)
{
    if (divisor < 1 || n_end > 0x80000000u) return -1;
    const FastDiv f = make_fastdiv(divisor);
    int64_t bad = 0;
    for (uint32_t n = 0; n < n_end; ++n) {
        uint32_t q, r;
        fdivmod(n, f, q, r);
        if (q != n / divisor || r != n % divisor) ++bad;
    }
    return bad;
}

}  // extern "C"
