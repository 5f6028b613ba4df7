// Internal declarations shared by the library's translation units: the error
// channel, device limits, the checked launch helper, and the per-file launch
// functions that the C entry points call.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "ftq.h"

namespace ftq {

constexpr int kQK = 32;
constexpr int kQ4Bytes = 18;
constexpr int kQ8Bytes = 36;

// Thread-local error text, returned by ftq_last_error().
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// Per-device limits, queried once per device.
struct DeviceLimits {
    int device = -1;
    int64_t max_grid_x = 0;       // blocks along x
    int64_t max_threads = 0;      // threads per block
    int64_t max_lds = 0;          // dynamic + static LDS bytes per block
    int cu_count = 0;
};
int device_limits(DeviceLimits* out);   // FTQ_OK or FTQ_ERR_HIP

int forced_block_threads();             // test hook value (0 = off)
// grouped-path kernel choice (ftq_debug_grouped_kernel; int8 MFMAs by default)
enum GroupedKernel { kGroupedI8 = 0, kGroupedF16 = 1, kGroupedF16Ws = 2 };
int grouped_kernel_variant();
int route_split_forced();               // test hook: bucketing in three kernels at any size

// Launch `kernel` with a 1-D grid, after checking the geometry against the
// device limits, and check the launch right after it is issued.  `name`
// identifies the kernel in error messages.
template <typename... KArgs, typename... Args>
int launch(const char* name, void (*kernel)(KArgs...), int64_t grid, int block, size_t lds,
           hipStream_t stream, Args... args)
{
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    int forced = forced_block_threads();
    if (forced > 0) block = forced;
    // AQL packets carry the grid in work-items per dimension as uint32.
    const int64_t items = grid * (int64_t)block;
    if (grid < 1 || grid > lim.max_grid_x || block < 1 || block > lim.max_threads ||
        items > (int64_t)UINT32_MAX || (int64_t)lds > lim.max_lds) {
        set_error("launch of %s rejected before issue: grid=(%lld,1,1) block=(%d,1,1) lds=%zu B "
                  "(device %d limits: grid.x<=%lld, block<=%lld, grid*block<=4294967295, lds<=%lld B)",
                  name, (long long)grid, block, lds, lim.device, (long long)lim.max_grid_x,
                  (long long)lim.max_threads, (long long)lim.max_lds);
        return FTQ_ERR_LAUNCH;
    }
    (void)hipGetLastError();   // errors of earlier, unrelated calls are not ours to report
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(block), lds, stream, args...);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        set_error("launch of %s failed: %s (%s) grid=(%lld,1,1) block=(%d,1,1) lds=%zu B",
                  name, hipGetErrorName(err), hipGetErrorString(err), (long long)grid, block, lds);
        return FTQ_ERR_LAUNCH;
    }
    return FTQ_OK;
}

// Number of workgroups for a grid-stride kernel: enough to fill the device
// several times over, never more than the work needs.
int64_t stride_grid(int64_t work_groups_needed, const DeviceLimits& lim, int per_cu = 16);

// ---- per-file launchers ------------------------------------------------------

int run_quantize_q8_1(const float* x, int64_t T, int64_t K, void* y, hipStream_t s);
int run_quantize_q4_0(const float* w, int64_t rows, int64_t K, void* y, hipStream_t s);

// Bucketing of pairs by expert (ids outside [0,E) go to the extra bucket E).
struct BucketPlan {
    int64_t pairs = 0;        // T * top_k
    int64_t buckets = 0;      // E + 1
    int64_t chunks = 0;       // ceil(pairs / kBucketChunk)
    int64_t tile_m = 0;       // rows per grouped tile (0: no tile table needed)
    // byte offsets inside the workspace
    int64_t off_counts = 0;   // int32 [buckets][chunks]: per-chunk counts, then sorted base positions
    int64_t off_offsets = 0;  // int32 [buckets + 1]: start slot of each bucket
    int64_t off_tiles = 0;    // int32 [buckets + 1]: first tile of each bucket
    int64_t off_sorted = 0;   // int32 [pairs]: pair ids grouped by bucket, ascending within one
    int64_t max_tiles = 0;    // grouped tiles at most (0: no tile table)
    int64_t off_tdesc = 0;    // int32x4 [max_tiles]: per tile {bucket, first slot, rows, 0}
    int64_t bytes = 0;
};
constexpr int kBucketChunk = 1024;   // pairs per wave in the counting and scatter passes
BucketPlan make_bucket_plan(int64_t pairs, int64_t E, int64_t tile_m);
int run_bucket(const int32_t* ids, int64_t E, const BucketPlan& plan, void* ws, hipStream_t s);

struct MoeArgs {
    const void* w;
    const void* a;
    const int32_t* ids;
    float* out;            // fp32 outputs, or
    int32_t* partials;     // integer partials when non-null
    int64_t E, N, K, T, top_k;
    int64_t act_div;       // activation row of pair p: p / act_div (top_k: per token; 1: per pair)
    int act;               // 0: plain output [T*k][N]; FTQ_ACT_*: act(gate) * up, [T*k][N/2]
    int wtype;             // weight block type (FTQ_W_*); the grouped path takes Q4_0, Q4_1 and Q8_0
};

// Gated activation of one fp32 value ("Current Bug: CuTeDSLMoERunner", Bug 6:
// SiLU; FreeToken PR #185, Problem: the tanh form of GELU), both as x times a
// logistic, x / (1 + e^-y): y = x for SiLU, and for GELU y = 2 sqrt(2/pi)
// (x + 0.044715 x^3), since (1 + tanh(z)) / 2 = 1 / (1 + e^-2z).  e^-y is one
// hardware exp2 of -y log2(e) and the quotient one hardware reciprocal: the
// relative error stays within a few units of the last place plus |y| units for
// the exponent's rounding, which the tests bound as 9 u (|act| + |x|).  Large
// |y| saturate cleanly: e^-y = inf gives x * 0, e^-y = 0 gives x.
__device__ __forceinline__ float gated_act(int act, float x)
{
    const float y = act == FTQ_ACT_SILU ? x : 1.5957691216057308f * (x + 0.044715f * x * x * x);
    const float e = __builtin_amdgcn_exp2f(-y * 1.4426950408889634f);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// GEMV path; `bucketed` selects the pair list from the workspace (else the
// kernel scans the ids itself).
int run_gemv(const MoeArgs& m, const BucketPlan* plan, const void* ws, hipStream_t s);

// The GEMV's on-chip plan, host arithmetic of the sizes alone: activation rows
// staged per pass, K blocks per segment (seg < K/32: rows are streamed in
// several K segments), LDS bytes and workgroups per CU.
struct GemvPlan {
    int64_t pc_cap = 0, seg = 0, lds = 0, per_cu = 0, item_base = 0, list_cap = 0;
    bool fits = false;   // false: a fused activation's whole row does not fit
};
GemvPlan plan_gemv(const MoeArgs& m, bool bucketed);
constexpr int64_t kGemvScanMaxPairs = 4096;

// Device helper.  Values every lane holds the same copy of (read from LDS or from global memory
// at a uniform address): moved to scalar registers so that loops over them are
// scalar loops.
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v)
{
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Grouped MFMA path.  Its workspace is the bucket plan's bytes.
int run_grouped(const MoeArgs& m, const BucketPlan& plan, void* ws, hipStream_t s);
int64_t grouped_tile_m(const MoeArgs& m);

// ftq_moe_q4_0_q8_1 with its validation, for entry points that supply the
// workspace themselves; and the workspace it needs (status: FTQ_OK or the
// validation error).
int moe_q4_0_q8_1_call(const void* w, const void* a, const int32_t* ids, float* out, int64_t E, int64_t N, int64_t K,
                       int64_t T, int64_t top_k, void* ws, size_t ws_bytes, int path, hipStream_t stream);
int64_t moe_workspace_need(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path, int* status);

// Top-k weighted combine of per-pair rows into per-token rows.
int run_combine_topk(const float* y, const float* gates, float* out, int64_t T, int64_t top_k, int64_t N,
                     hipStream_t s);

}  // namespace ftq
