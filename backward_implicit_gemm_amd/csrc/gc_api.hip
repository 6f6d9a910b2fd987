// gc_api.hip -- the C ABI declared in include/gc.h: argument validation, the
// output-size closed form, workspace sizing and kernel selection.  All
// validation happens before the first HIP call, so the error paths are
// testable on a machine without a GPU.
#include <limits.h>
#include <stdarg.h>
#include <stdio.h>

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

// Compute units and XCDs of the current device, queried once per device.
// Without a usable device (a host-only process asking for workspace sizes or
// plan names) the MI355X values are used: 256 CUs in 8 XCDs.
void set_device(Geom &g)
{
    constexpr int kMaxDev = 64;
    static std::mutex m;
    static int known[kMaxDev][2];
    static bool have[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();   // leave no error behind for the next call
        g.ncu = 256;
        g.nxcd = 8;
        return;
    }
    std::lock_guard<std::mutex> lk(m);
    if (!have[dev]) {
        int ncu = 0, nxcd = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            ncu < 1)
            ncu = 256;
        if (hipDeviceGetAttribute(&nxcd, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
            nxcd < 1 || ncu % nxcd)
            nxcd = 1;
        (void)hipGetLastError();
        known[dev][0] = ncu;
        known[dev][1] = nxcd;
        have[dev] = true;
    }
    g.ncu = known[dev][0];
    g.nxcd = known[dev][1];
}

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
    if (g) {
        *g = make_geom(d->B, d->IC, d->H, d->W, d->OC, d->KH, d->KW, d->stride);
        set_device(*g);
    }
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

// Plans depend only on the geometry and the device's CU and XCD counts, and
// some take a search (the forward's LDS pitch) that costs far more host time
// than a launch, so each planner's answers are kept per (geometry, device
// shape), one table per planner (two planners may share a plan type).
// Thread-safe; a full table overwrites its entries round-robin.
template <typename P, bool (*Planner)(const Geom &, P &)>
bool cached_plan(const Geom &g, P &out)
{
    struct Entry {
        int key[10];
        bool ok;
        P plan;
    };
    constexpr int kSlots = 64;
    static std::mutex m;
    static Entry table[kSlots];
    static int used = 0, next = 0;
    const int key[10] = {g.B, g.IC, g.H, g.W, g.OC, g.KH, g.KW, g.S, g.ncu, g.nxcd};
    {
        std::lock_guard<std::mutex> lk(m);
        for (int i = 0; i < used; ++i)
            if (std::equal(key, key + 10, table[i].key)) {
                if (table[i].ok) out = table[i].plan;
                return table[i].ok;
            }
    }
    P p{};
    const bool ok = Planner(g, p);
    std::lock_guard<std::mutex> lk(m);
    Entry &e = table[used < kSlots ? used++ : (next++ % kSlots)];
    std::copy(key, key + 10, e.key);
    e.ok = ok;
    e.plan = p;
    if (ok) out = p;
    return ok;
}

bool fwd_f32_ws_plan(const Geom &g, FwdWsPlan &p)
{
    return use_ig() && cached_plan<FwdWsPlan, plan_fwd_ws_f32>(g, p);
}
bool fwd_bf16_ws_plan(const Geom &g, FwdWsPlan &p)
{
    return use_ig() && cached_plan<FwdWsPlan, plan_fwd_ws_bf16>(g, p);
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
bool bwd_fused_f32_plan(const Geom &g, BwdFusedF32Plan &p)
{
    return use_ig() && cached_plan<BwdFusedF32Plan, plan_bwd_fused_f32>(g, p);
}
size_t round256(size_t n) { return (n + 255) & ~size_t(255); }
bool wgrad_f32_rf_plan(const Geom &g, WgradRfPlan &p)
{
    return use_ig() && cached_plan<WgradRfPlan, plan_wgrad_rf_f32>(g, p);
}
bool wgrad_bf16_bias_plan(const Geom &g, WgradBfPlan &p)
{
    return use_ig() && cached_plan<WgradBfPlan, plan_wgrad_ig_bf16_bias>(g, p);
}
bool wgrad_f32_rf_bias_plan(const Geom &g, WgradRfPlan &p)
{
    return use_ig() && cached_plan<WgradRfPlan, plan_wgrad_rf_f32_bias>(g, p);
}
bool wgrad_plan(const Geom &g, WgradIgPlan &p)
{
    return use_ig() && cached_plan<std::remove_reference_t<decltype(p)>, plan_wgrad_ig_f32>(g, p);
}

// ---------------------------------------------------------------------------
// Kernel selection.  Each entry point asks select_* which kernel family runs
// a problem, in a fixed order of preference, and gc_conv_plan_name() reports
// the same choice, so tests can pin which kernel every tested shape runs.
// ---------------------------------------------------------------------------
enum class FwdKind { WsF32, WsBf16, Generic };
struct FwdSel {
    FwdKind k;
    FwdWsPlan ws;
};
FwdSel select_fwd(const Geom &g, int dtype)
{
    FwdSel s{};
    if (dtype == GC_F32)
        s.k = fwd_f32_ws_plan(g, s.ws) ? FwdKind::WsF32 : FwdKind::Generic;
    else
        s.k = fwd_bf16_ws_plan(g, s.ws) ? FwdKind::WsBf16 : FwdKind::Generic;
    return s;
}

enum class DgradKind { IgBf16, RfF32, IgF32Mfma, Generic };
struct DgradSel {
    DgradKind k;
    DgradBfPlan bf;
    DgradIgPlan ig;
};
DgradSel select_dgrad(const Geom &g, int dtype)
{
    DgradSel s{};
    if (dtype == GC_BF16 && dgrad_bf16_plan(g, s.bf)) s.k = DgradKind::IgBf16;
    else if (dtype == GC_F32 && dgrad_f32_rf_plan(g, s.bf)) s.k = DgradKind::RfF32;
    else if (dgrad_plan(g, s.ig)) s.k = DgradKind::IgF32Mfma;
    else s.k = DgradKind::Generic;
    return s;
}

enum class WgradKind { IgBf16, RfF32, IgF32Mfma, Generic };
struct WgradSel {
    WgradKind k;
    WgradBfPlan bf;
    WgradRfPlan rf;
    WgradIgPlan ig;
    int splits;   // partial tiles of the IgF32Mfma and Generic kinds
};
WgradSel select_wgrad(const Geom &g, int dtype)
{
    WgradSel s{};
    if (dtype == GC_BF16 && wgrad_bf16_plan(g, s.bf)) s.k = WgradKind::IgBf16;
    else if (dtype == GC_F32 && wgrad_f32_rf_plan(g, s.rf)) s.k = WgradKind::RfF32;
    else if (wgrad_plan(g, s.ig)) {
        s.k = WgradKind::IgF32Mfma;
        s.splits = s.ig.splits;
    } else {
        s.k = WgradKind::Generic;
        s.splits = wgrad_generic_splits(g);
    }
    return s;
}

// wgrad with the bias gradient: the bias as one more column of the wgrad
// tiles where the kernels have it (bf16, and the fp32 image-quad kernel),
// else wgrad and the separate bias-gradient kernels.
enum class WgradBiasKind { IgBf16, RfF32, Separate };
struct WgradBiasSel {
    WgradBiasKind k;
    WgradBfPlan bf;
    WgradRfPlan rf;
};
WgradBiasSel select_wgrad_bias(const Geom &g, int dtype)
{
    WgradBiasSel s{};
    if (dtype == GC_BF16 && wgrad_bf16_bias_plan(g, s.bf)) s.k = WgradBiasKind::IgBf16;
    else if (dtype == GC_F32 && wgrad_f32_rf_bias_plan(g, s.rf)) s.k = WgradBiasKind::RfF32;
    else s.k = WgradBiasKind::Separate;
    return s;
}

// Appends printf-style text to buf (bounded by n, always NUL-terminated).
void append(char *buf, size_t n, size_t &at, const char *fmt, ...)
    __attribute__((format(printf, 4, 5)));
void append(char *buf, size_t n, size_t &at, const char *fmt, ...)
{
    if (at >= n) return;
    va_list ap;
    va_start(ap, fmt);
    const int k = vsnprintf(buf + at, n - at, fmt, ap);
    va_end(ap);
    if (k > 0) at = std::min(n - 1, at + size_t(k));
}

// Names: the kernel family and its compile-time instance in <>, then the
// launch parameters of the plan.
void name_fwd(const FwdSel &s, char *buf, size_t n, size_t &at)
{
    switch (s.k) {
    case FwdKind::WsF32:
        append(buf, n, at, "fwd_ws_f32<NWM=%d,MB=%d,TS=%d,NCG=%d,CPP=%d,LO=%d> G=%d ntile=%d", s.ws.NWM,
               s.ws.MB, s.ws.TS, s.ws.NCG, s.ws.CPP, s.ws.lo, s.ws.G, s.ws.ntile);
        break;
    case FwdKind::WsBf16:
        append(buf, n, at, "fwd_ws_bf16<NBW=%d,MB=%d,TS=%d,NCG=%d,CPP=%d> G=%d ntile=%d", s.ws.NBW,
               s.ws.MB, s.ws.TS, s.ws.NCG, s.ws.CPP, s.ws.G, s.ws.ntile);
        break;
    case FwdKind::Generic: append(buf, n, at, "igemm_generic_fwd"); break;
    }
}

void name_dgrad_bf(const DgradBfPlan &p, char *buf, size_t n, size_t &at)
{
    append(buf, n, at, "dgrad_ig_bf16<MB=%d,KS=%d,TAPS=%d,NBW=%d> G=%d CC=%d", p.MB, p.KS, p.TAPS,
           p.NBW, p.G, p.CC);
}

void name_dgrad(const DgradSel &s, char *buf, size_t n, size_t &at)
{
    switch (s.k) {
    case DgradKind::IgBf16: name_dgrad_bf(s.bf, buf, n, at); break;
    case DgradKind::RfF32:
        append(buf, n, at, "dgrad_rf_f32<MB=%d,KS4=%d,TAPS=%d> G=%d CC=%d", s.bf.MB, s.bf.KS,
               s.bf.TAPS, s.bf.G, s.bf.CC);
        break;
    case DgradKind::IgF32Mfma:
        append(buf, n, at, "dgrad_ig_f32<MB=%d> G=%d CC=%d", s.ig.MB, s.ig.G, s.ig.CC);
        break;
    case DgradKind::Generic: append(buf, n, at, "igemm_generic_dgrad"); break;
    }
}

void name_wgrad(const WgradSel &s, char *buf, size_t n, size_t &at)
{
    switch (s.k) {
    case WgradKind::IgBf16:
        append(buf, n, at, "wgrad_ws_bf16<NSTEP=%d,JW=%d> ncol=%d splits=%d", s.bf.NSTEP, s.bf.JW,
               s.bf.ncol, s.bf.splits);
        break;
    case WgradKind::RfF32:
        append(buf, n, at, "wgrad_rf_f32<NBWV=%d> chunks=%d splits=%d", s.rf.NBWV, s.rf.chunks,
               s.rf.splits);
        break;
    case WgradKind::IgF32Mfma:
        append(buf, n, at, "wgrad_ig_f32<MBW=%d> G=%d splits=%d", s.ig.MBW, s.ig.G, s.splits);
        break;
    case WgradKind::Generic: append(buf, n, at, "igemm_generic_wgrad splits=%d", s.splits); break;
    }
}
// Scratch memory of gc_conv_fwd_noalloc: a file-scope device array (each
// GPU the library runs on holds its own copy until the process ends), used
// for the forward's packed weights.  Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol); it passes the
// device address hipGetSymbolAddress gives for the current device, taken
// once per device.
constexpr size_t kNoallocScratchBytes = size_t(2) << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// The current device's address of `scratch`, or nullptr (and *err set) if
// it cannot be had.
void *scratch_address(hipError_t *err)
{
    constexpr int kMaxDev = 64;
    static std::mutex m;
    static void *addr[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDev)) e = hipErrorInvalidDevice;
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(m);
    if (!addr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = ptr;
    }
    return addr[dev];
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
        const FwdSel s = select_fwd(g, dtype);
        return s.k == FwdKind::Generic ? 0 : s.ws.ws_bytes;
    }
    case GC_OP_BWD_DATA: {
        const DgradSel s = select_dgrad(g, dtype);
        return s.k == DgradKind::IgBf16 ? s.bf.ws_bytes : 0;
    }
    case GC_OP_BWD_WEIGHT: {
        const WgradSel s = select_wgrad(g, dtype);
        if (s.k == WgradKind::IgBf16) return s.bf.ws_bytes;
        if (s.k == WgradKind::RfF32) return s.rf.ws_bytes;
        return size_t(s.splits) * g.OC * g.K * sizeof(float);
    }
    case GC_OP_BWD_BIAS: return bias_grad_ws_bytes(g);
    case GC_OP_BWD_WEIGHT_BIAS: {
        const WgradBiasSel s = select_wgrad_bias(g, dtype);
        if (s.k == WgradBiasKind::IgBf16) return s.bf.ws_bytes;
        if (s.k == WgradBiasKind::RfF32) return s.rf.ws_bytes;
        // wgrad's workspace, then the bias gradient's at the next 256-byte boundary
        return round256(gc_conv_workspace_bytes(GC_OP_BWD_WEIGHT, d, dtype)) + bias_grad_ws_bytes(g);
    }
    case GC_OP_BWD: {
        BwdFusedBfPlan p;
        if (dtype == GC_BF16 && bwd_fused_plan(g, p)) return p.ws_bytes;
        BwdFusedF32Plan pf;
        if (dtype == GC_F32 && bwd_fused_f32_plan(g, pf)) return pf.ws_bytes;
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
    const FwdSel sel = select_fwd(g, dtype);
    if (sel.k != FwdKind::Generic) {
        if (!workspace || ws_bytes < sel.ws.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
    }
    switch (sel.k) {
    case FwdKind::WsF32:
        return hip_status(launch_fwd_ws_f32(g, sel.ws, x, w, bias, y, workspace, relu, s));
    case FwdKind::WsBf16:
        return hip_status(launch_fwd_ws_bf16(g, sel.ws, x, w, bias, y, workspace, relu, s));
    case FwdKind::Generic: break;
    }
    return hip_status(dtype == GC_F32 ? launch_fwd_generic<float>(g, x, w, bias, y, relu, s)
                                      : launch_fwd_generic<bf16_t>(g, x, w, bias, y, relu, s));
}

int gc_conv_fwd(const void *x, const void *w, void *y, void *workspace, size_t ws_bytes,
                const gc_conv_desc *d, int relu, int dtype, void *stream)
{
    return conv_fwd(x, w, nullptr, y, workspace, ws_bytes, d, relu, dtype, stream);
}

int gc_conv_fwd_noalloc(const void *x, const void *w, void *y, const gc_conv_desc *d, int relu,
                        int dtype, void *stream)
{
    // the same checks as gc_conv_fwd, then the workspace the plan needs
    // against the static scratch, all before any HIP call
    Geom g;
    const int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!x || !w || !y) return GC_ERR_INVALID_ARG;
    if (!aligned(x, dtype) || !aligned(w, dtype) || !aligned(y, dtype)) return GC_ERR_INVALID_ARG;
    const size_t need = gc_conv_workspace_bytes(GC_OP_FWD, d, dtype);
    if (need > kNoallocScratchBytes) return GC_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need) {
        hipError_t e = hipSuccess;
        ws = scratch_address(&e);
        if (!ws) return hip_status(e);
    }
    // the packed weights are written in full by the call before they are
    // read, so nothing in the scratch needs clearing
    return conv_fwd(x, w, nullptr, y, ws, need ? kNoallocScratchBytes : 0, d, relu, dtype, stream);
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
    const DgradSel sel = select_dgrad(g, dtype);
    switch (sel.k) {
    case DgradKind::IgBf16:
        if (!workspace || ws_bytes < sel.bf.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
        return hip_status(launch_dgrad_ig_bf16(g, sel.bf, dy, w, y_mask, dx, workspace, relu, s));
    case DgradKind::RfF32:
        return hip_status(launch_dgrad_rf_f32(g, sel.bf, dy, w, y_mask, dx, relu, s));
    case DgradKind::IgF32Mfma:
        return hip_status(dtype == GC_F32
                              ? launch_dgrad_ig<float>(g, sel.ig, dy, w, y_mask, dx, relu, s)
                              : launch_dgrad_ig<bf16_t>(g, sel.ig, dy, w, y_mask, dx, relu, s));
    case DgradKind::Generic: break;
    }
    return hip_status(dtype == GC_F32
                          ? launch_dgrad_generic<float>(g, dy, w, y_mask, dx, relu, s)
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
    const WgradSel sel = select_wgrad(g, dtype);
    if (sel.k == WgradKind::IgBf16) {
        if (!workspace || ws_bytes < sel.bf.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
        return hip_status(launch_wgrad_ig_bf16(g, sel.bf, x, dy, y_mask, dw, nullptr, workspace, relu, s));
    }
    if (sel.k == WgradKind::RfF32) {
        if (!workspace || ws_bytes < sel.rf.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
        return hip_status(launch_wgrad_rf_f32(g, sel.rf, x, dy, y_mask, dw, nullptr, workspace, relu, s));
    }
    const int splits = sel.splits;
    const size_t need = size_t(splits) * g.OC * g.K * sizeof(float);
    if (need && (!workspace || ws_bytes < need)) return GC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
    float *part = static_cast<float *>(workspace);
    const bool ig = sel.k == WgradKind::IgF32Mfma;
    hipError_t e;
    if (dtype == GC_F32) {
        e = ig ? launch_wgrad_ig<float>(g, sel.ig, x, dy, y_mask, part, relu, s)
               : launch_wgrad_generic<float>(g, x, dy, y_mask, part, splits, relu, s);
        if (e == hipSuccess) e = launch_wgrad_reduce<float>(part, dw, splits, g.OC * g.K, s);
    } else {
        e = ig ? launch_wgrad_ig<bf16_t>(g, sel.ig, x, dy, y_mask, part, relu, s)
               : launch_wgrad_generic<bf16_t>(g, x, dy, y_mask, part, splits, relu, s);
        if (e == hipSuccess) e = launch_wgrad_reduce<bf16_t>(part, dw, splits, g.OC * g.K, s);
    }
    return hip_status(e);
}

int gc_conv_bwd_weight_bias(const void *x, const void *dy, const void *y_mask, void *dw, void *db,
                            void *workspace, size_t ws_bytes, const gc_conv_desc *d, int relu,
                            int dtype, void *stream)
{
    Geom g;
    int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || (relu != 0 && relu != 1)) return GC_ERR_INVALID_ARG;
    if (!x || !dy || !dw || !db) return GC_ERR_INVALID_ARG;
    if ((relu == 1) != (y_mask != nullptr)) return GC_ERR_INVALID_ARG;
    if (!aligned(x, dtype) || !aligned(dy, dtype) || !aligned(dw, dtype) || !aligned(db, dtype) ||
        (y_mask && !aligned(y_mask, dtype)))
        return GC_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const WgradBiasSel sel = select_wgrad_bias(g, dtype);
    if (sel.k == WgradBiasKind::IgBf16) {
        if (!workspace || ws_bytes < sel.bf.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
        return hip_status(launch_wgrad_ig_bf16(g, sel.bf, x, dy, y_mask, dw, db, workspace, relu, s));
    }
    if (sel.k == WgradBiasKind::RfF32) {
        if (!workspace || ws_bytes < sel.rf.ws_bytes) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return GC_ERR_WORKSPACE;
        return hip_status(launch_wgrad_rf_f32(g, sel.rf, x, dy, y_mask, dw, db, workspace, relu, s));
    }
    // no bias column: wgrad, then the bias gradient, each in its part of the workspace
    const size_t ww = gc_conv_workspace_bytes(GC_OP_BWD_WEIGHT, d, dtype);
    const size_t off = round256(ww);
    const size_t need = off + bias_grad_ws_bytes(g);
    if (!workspace || ws_bytes < need) return GC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
    st = gc_conv_bwd_weight(x, dy, y_mask, dw, ww ? workspace : nullptr, ww, d, relu, dtype, stream);
    if (st != GC_OK) return st;
    return gc_conv_bwd_bias(dy, y_mask, db, static_cast<char *>(workspace) + off, ws_bytes - off, d,
                            relu, dtype, stream);
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
    BwdFusedF32Plan ff;
    if (dtype == GC_F32 && bwd_fused_f32_plan(g, ff)) {
        if (ff.ws_bytes && (!workspace || ws_bytes < ff.ws_bytes)) return GC_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256) return GC_ERR_WORKSPACE;
        return hip_status(launch_bwd_fused_f32(g, ff, x, w, dy, y_mask, dx, dw, workspace, relu,
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

int gc_conv_plan_name(int op, const gc_conv_desc *d, int dtype, char *buf, size_t buf_bytes)
{
    Geom g;
    const int st = check_desc(d, &g);
    if (st != GC_OK) return st;
    if (!valid_dtype(dtype) || !buf || buf_bytes == 0) return GC_ERR_INVALID_ARG;
    size_t at = 0;
    buf[0] = '\0';
    switch (op) {
    case GC_OP_FWD: name_fwd(select_fwd(g, dtype), buf, buf_bytes, at); break;
    case GC_OP_BWD_DATA: name_dgrad(select_dgrad(g, dtype), buf, buf_bytes, at); break;
    case GC_OP_BWD_WEIGHT: name_wgrad(select_wgrad(g, dtype), buf, buf_bytes, at); break;
    case GC_OP_BWD_BIAS: append(buf, buf_bytes, at, "bias_partials+bias_final"); break;
    case GC_OP_BWD_WEIGHT_BIAS: {
        const WgradBiasSel s = select_wgrad_bias(g, dtype);
        WgradSel w{};
        if (s.k == WgradBiasKind::IgBf16) {
            w.k = WgradKind::IgBf16;
            w.bf = s.bf;
        } else if (s.k == WgradBiasKind::RfF32) {
            w.k = WgradKind::RfF32;
            w.rf = s.rf;
        } else {
            w = select_wgrad(g, dtype);
        }
        name_wgrad(w, buf, buf_bytes, at);
        append(buf, buf_bytes, at, s.k == WgradBiasKind::Separate ? " + bias_partials+bias_final"
                                                                  : " +bias column");
        break;
    }
    case GC_OP_BWD: {
        BwdFusedBfPlan fp;
        if (dtype == GC_BF16 && bwd_fused_plan(g, fp)) {
            append(buf, buf_bytes, at, "bwd_fused_bf16 fuse_main=%d: ", fp.fuse_main);
            name_dgrad_bf(fp.d, buf, buf_bytes, at);
            append(buf, buf_bytes, at, " + ");
            WgradSel w{};
            w.k = WgradKind::IgBf16;
            w.bf = fp.w;
            name_wgrad(w, buf, buf_bytes, at);
        } else if (BwdFusedF32Plan ff; dtype == GC_F32 && bwd_fused_f32_plan(g, ff)) {
            append(buf, buf_bytes, at, "bwd_fused_f32: ");
            DgradSel d{};
            d.k = DgradKind::RfF32;
            d.bf = ff.d;
            name_dgrad(d, buf, buf_bytes, at);
            append(buf, buf_bytes, at, " + ");
            WgradSel w{};
            w.k = WgradKind::RfF32;
            w.rf = ff.w;
            name_wgrad(w, buf, buf_bytes, at);
        } else {
            name_dgrad(select_dgrad(g, dtype), buf, buf_bytes, at);
            append(buf, buf_bytes, at, " + ");
            name_wgrad(select_wgrad(g, dtype), buf, buf_bytes, at);
        }
        break;
    }
    default: return GC_ERR_INVALID_ARG;
    }
    return GC_OK;
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
