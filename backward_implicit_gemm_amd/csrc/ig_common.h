// ig_common.h -- pieces shared by the image-group kernels: vector global
// loads at any element alignment, and the per-call tiling plans.
//
// An image-group kernel gives each workgroup whole images (or a split of the
// reduction for wgrad) so that the small spatial extent of the policy-network
// layers (OH*OW = 12 or 2 outputs per image) never leaves a tile mostly empty,
// and stages contiguous NCHW slabs instead of gathering element by element.
#pragma once

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "gc_common.h"

namespace gc {

// Raises a kernel's dynamic-LDS limit to the full 160 KiB once per (device,
// kernel); every later launch of it, with any LDS size up to that, needs no
// further attribute call.
inline hipError_t allow_max_lds(const void *fn)
{
    static std::mutex m;
    static std::vector<std::pair<int, const void *>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(m);
    for (const auto &d : done)
        if (d.first == dev && d.second == fn) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess) done.emplace_back(dev, fn);
    return e;
}

// A small thread-safe memo for planner searches whose answer does not depend
// on the batch size (LDS pitch choices), keyed by up to 12 ints.  A full
// table overwrites its entries round-robin.
template <typename V, int N = 64>
class SearchMemo {
  public:
    template <typename F>
    V get(const int (&key)[12], F compute)
    {
        {
            std::lock_guard<std::mutex> lk(m_);
            for (int i = 0; i < used_; ++i)
                if (std::equal(key, key + 12, e_[i].key)) return e_[i].v;
        }
        const V v = compute();
        std::lock_guard<std::mutex> lk(m_);
        Entry &e = e_[used_ < N ? used_++ : (next_++ % N)];
        std::copy(key, key + 12, e.key);
        e.v = v;
        return v;
    }

  private:
    struct Entry {
        int key[12];
        V v;
    };
    std::mutex m_;
    Entry e_[N];
    int used_ = 0, next_ = 0;
};

// Four consecutive elements as fp32 from an element-aligned global address:
// one 16-byte load for fp32 storage, one 8-byte load widened exactly for
// bf16 storage.
// Component i (0..3) of a float4, with i a compile-time constant after
// unrolling.
__device__ __forceinline__ float comp(const float4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float4 ld4_f32(const float *p)
{
    float4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}
__device__ __forceinline__ float4 ld4_f32(const bf16_t *p)
{
    uint2 u;
    __builtin_memcpy(&u, p, sizeof(u));
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

// 16-byte load from a 4-byte-aligned global address.  The compiler emits a
// single global_load_dwordx4 for this copy (the HSA runtime runs gfx9 parts in
// unaligned-access mode); callers keep all four elements inside the tensor.
__device__ __forceinline__ float4 ldg4_any(const float *p)
{
    float4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

constexpr int IG_NT = 256;   // threads per workgroup (4 waves)

// Buffer resource over a whole tensor of `bytes` bytes (< 2^31): a load
// whose offset is at or past the end returns zeros, so staging loads need no
// branches for images past the batch or channels past the tensor.  Word 3
// selects the 32-bit data format of the gfx9 buffer descriptor, with no
// swizzle and no index stride.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, int(bytes), 0x00020000);
}
// 16 bytes at byte offset `off` of the tensor (zeros past its end)
__device__ __forceinline__ float4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    float4 f;
    __builtin_memcpy(&f, &v, 16);
    return f;
}
__device__ __forceinline__ uint4 bload16u(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    uint4 u;
    __builtin_memcpy(&u, &v, 16);
    return u;
}
// 16 bytes at byte offset voff + soff, soff wave-uniform (a scalar register
// or a constant, so a sequence of loads from one base costs no vector
// registers for addresses)
__device__ __forceinline__ float4 bload16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    float4 f;
    __builtin_memcpy(&f, &v, 16);
    return f;
}
__device__ __forceinline__ uint4 bload16us(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    uint4 u;
    __builtin_memcpy(&u, &v, 16);
    return u;
}
// 4 bytes at byte offset voff + soff, soff wave-uniform (zeros past the end)
__device__ __forceinline__ float bload4s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
// store 4 bytes at byte offset voff + soff; a store whose voff alone is at
// or past the end of the tensor is dropped
__device__ __forceinline__ void bstore4s(__amdgpu_buffer_rsrc_t r, float v, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}
constexpr uint32_t kOffNone = 0xFFFFFFF0u;   // an offset past the end of every tensor

// s_waitcnt vmcnt(0): every vector memory operation this wave has issued has
// completed.  Placed where only loads issued long ago are outstanding, it
// retires them before later stores are issued, so a later use of the loaded
// registers does not wait for those stores as well.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------- forward --
// MFMA steps of the fp32 forward per 16-channel block, phase by phase: a
// phase stages ncg = min(CPP, NCG - ph*CPP) channel groups; each group takes
// TSF tap steps (taps 4s .. 4s+3 on the four lane groups), TSF = TS, or TS-1
// when `lo`: then KH*KW = 4*(TS-1) + 1 and the last tap of the phase's groups
// is covered by ceil(ncg/4) shared steps, lane group q taking group 4l+q of
// the phase (no zero-padded taps beyond the last step's unused lanes).
struct FwdF32Steps {
    int NCG, CPP, TS, lo;
    __host__ __device__ constexpr int tsf() const { return lo ? TS - 1 : TS; }
    __host__ __device__ constexpr int nph() const { return (NCG + CPP - 1) / CPP; }
    __host__ __device__ constexpr int ncg(int ph) const { return NCG - ph * CPP < CPP ? NCG - ph * CPP : CPP; }
    __host__ __device__ constexpr int nfull(int ph) const { return ncg(ph) * tsf(); }
    __host__ __device__ constexpr int nsteps(int ph) const { return nfull(ph) + (lo ? (ncg(ph) + 3) / 4 : 0); }
    __host__ __device__ constexpr int base(int ph) const
    {
        int b = 0;
        for (int i = 0; i < ph; ++i) b += nsteps(i);
        return b;
    }
    __host__ __device__ constexpr int nfrag() const { return base(nph()); }
};
// Forward with loader and MFMA waves (fwd_ws_bf16.hip, fwd_ws_f32.hip).
struct FwdWsPlan {
    int NWM;      // MFMA waves (as many loader waves; fp32 only, bf16 uses 4)
    int NBW;      // 16-channel blocks per MFMA wave
    int G;        // images per workgroup
    int MB;       // 16-row M blocks
    int TS;       // tap steps: ceil(KH*KW/4)
    int WP, IS;   // LDS pixel slots per image row / per image
    int nblk;     // pixel blocks per image plane (8 pixels bf16, 4 fp32)
    int NCG;      // channel groups (8 channels bf16, 4 fp32)
    int CPP;      // channel groups per staging phase
    int ntile;    // column tiles
    int lo;       // fp32: the last tap of every channel group in shared steps (KH*KW % 4 == 1)
    int ystage;   // bf16: output staged through LDS for 16-byte stores
    size_t lds;       // the whole x tile (bf16), two phase buffers (fp32)
    size_t ws_bytes;  // packed weights
};

// ---------------------------------------------------------------- d_input --
// bf16 d_input on bf16 MFMA (dgrad_ig_bf16.hip).
struct DgradBfPlan {
    int NW;       // waves per workgroup (they split each chunk's column blocks)
    int G;        // images per workgroup, a multiple of 4
    int MB;       // 16-row blocks over the G*P rows m = p*G + img
    int KS;       // 32-channel steps over OC (zero-padded)
    int TAPS;     // register slots for the taps of one input pixel
    int NBW;      // column blocks per wave per chunk, ceil(NBC / NW)
    int GP;       // gather passes per chunk (planes CC*G/4 <= GP * gather threads per pixel)
    int CC;       // input channels per chunk
    int NBC;      // 16-column blocks per chunk, ceil(CC*KH*KW / 16)
    int nchunks;  // ceil(IC / CC)
    int cgroups;  // workgroups along the chunks
    int cpg;      // chunks per workgroup
    int RP;       // dcol column pitch in floats (MB*16 + 4)
    int OCP;      // dz row pitch in bf16 elements (32*KS + 8)
    int dz_bytes; // LDS bytes of the dz tile
    int ORUN;     // dx tile row (one image's chunk, CC*H*W) rounded up to 8 elements
    size_t lds;       // dz tile + double-buffered dcol + double-buffered dx tile
    size_t ws_bytes;  // packed weights
};

struct DgradIgPlan {
    int NW;       // waves per workgroup (they split the dcol columns)
    int G;        // images per workgroup
    int MB;       // 16-row M blocks over G*P rows
    int CC;       // input channels per chunk
    int NCH;      // CC*KK dcol columns per chunk
    int NBT;      // 16-column blocks per chunk (ceil(NCH/16))
    int NBW;      // blocks per wave (ceil(NBT/4))
    int OCS;      // output channels per weight sub-chunk (multiple of 4)
    int nsub;     // ceil(OC/OCS)
    int OCP;      // OC rounded up to OCS multiple
    int DZP;      // LDS row stride of dz rows
    int WCP;      // LDS row stride of the weight sub-chunk
    int DCP;      // LDS row stride of dcol
    int TH, TW;   // max taps per input row / column: ceil(KH/S), ceil(KW/S)
    int nchunks;  // ceil(IC/CC)
    int cgroups;  // channel groups along grid.y
    int cpg;      // chunks per channel group
    int WV;       // float4 staging loads per thread for a weight sub-chunk
    size_t lds;
};

// ---------------------------------------------------------------- wgrad ----
// bf16 wgrad on bf16 MFMA (wgrad_ig_bf16.hip).
struct WgradBfPlan {
    int NSTEP;    // MFMA steps per 8-image group, PP / 4
    int JW;       // 16-column blocks per MFMA wave: tiles of 64*JW columns
    int bias;     // also the bias gradient: column K of the tiles, with x = 1
    int NP;       // columns per partial row: K, or K+1 rounded up to 4 with the bias
    int PP;       // output positions padded to a multiple of 4
    int CCW;      // input channels staged per column tile (widest span)
    int nblk;     // 8-pixel blocks per channel plane
    int HWP;      // LDS pixel slots per staged channel (nblk * 8)
    int ncol;     // column tiles over IC*KH*KW
    int ngroups;  // 8-image groups, ceil(B / 8)
    int gps;      // groups per split
    int splits;   // workgroup rows (partial tiles)
    size_t lds;       // double-buffered x and dz stages
    size_t dz_bytes;  // regrouped dz at the front of the workspace
    size_t ws_bytes;  // dz_bytes + splits * OC * NP fp32 partials
};

// fp32 wgrad with image-quad staging (wgrad_rf_f32.hip).
struct WgradRfPlan {
    int NBWV;     // 16-column blocks per wave
    int MBLK;     // 16-row oc blocks, ceil(OC / 16)
    int WN;       // waves per oc block (they split the column blocks)
    int NBW;      // 16-column blocks per workgroup, WN * NBWV
    int chunks;   // column chunks, ceil(ceil(K / 16) / NBW)
    int NQ;       // 4-image quads, ceil(B / 4)
    int QB;       // quads per staging phase
    int QPS;      // quads per split
    int splits;   // partial tiles
    int SPP;      // 4-step MFMA blocks per phase, ceil(QB * P / 4)
    int CCS;      // channels staged per chunk (widest span)
    int XU;       // x staging units per quad, ceil(CCS * H * W / 4)
    int DU;       // dz staging units per quad, ceil(OC * P / 4)
    int WP, IS;   // x LDS slots per pixel row / per channel
    int OCP;      // dz LDS slots per output position (>= OC)
    int bufsz;    // 16-byte slots per LDS buffer (x, dz, one zero slot)
    int bias;     // also the bias gradient: column K of the tiles, with x = 1
    int NP;       // columns per partial row: K, or K+1 rounded up to 4 with the bias
    size_t lds;
    size_t ws_bytes;   // splits * OC * NP fp32 partials
};

struct WgradIgPlan {
    int NW;       // waves per workgroup: 4 split OC, NW/4 split the k tile
    int G;        // images per stage
    int R4;       // stage rows G*P rounded up to 4 (one fp32 MFMA step)
    int RP;       // LDS row stride of the transposed dz stage
    int MBW;      // 16-row oc blocks per wave (OC <= 64*MBW)
    int NBK;      // 16-column k blocks per tile (NBK/(NW/4) per wave)
    int BNK;      // 16*NBK
    int nkt;      // k tiles
    int NCHS;     // max channels a k tile spans
    int XSS;      // LDS floats per image of the x stage (NCHS*HW rounded up to 4)
    int GS;       // images per split
    int splits;
    int DV, XV;   // staging loads per thread (dz scalars, x float4)
    size_t lds;
};

// bf16 backward in three or four launches (bwd_fused_bf16.hip): the d_input
// and wgrad plans it runs, and where wgrad's part of the workspace starts.
struct BwdFusedBfPlan {
    DgradBfPlan d;
    WgradBfPlan w;
    size_t ws_w_offset;   // d.ws_bytes rounded up to 256
    size_t ws_bytes;      // ws_w_offset + w.ws_bytes
    int fuse_main;        // both main kernels in one grid
};

// fp32 backward in two launches (bwd_fused_f32.hip): the d_input and wgrad
// workgroups in one grid, then the reduction.
struct BwdFusedF32Plan {
    DgradBfPlan d;
    WgradRfPlan w;
    size_t ws_bytes;      // w.ws_bytes (the fp32 d_input needs no workspace)
};

}  // namespace gc
