// The C entry points of libftq: argument validation, path choice, workspace
// planning and dispatch.  No allocation, no synchronisation, no readback.
#include <cstdarg>
#include <mutex>

#include "ftq_internal.h"

namespace ftq {

namespace {
thread_local std::string g_error;
thread_local int g_forced_threads = 0;
thread_local int g_grouped_variant = kGroupedI8;

constexpr int kMaxDevices = 64;
std::mutex g_lim_mu;
DeviceLimits g_lim[kMaxDevices];

constexpr int64_t kMaxExperts = 4095;      // bucket tables live in LDS
constexpr int64_t kMaxPairs = INT32_MAX;   // pair ids are stored as int32

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
}  // namespace

void set_error(const char* fmt, ...)
{
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
}

void clear_error() { g_error.clear(); }

int forced_block_threads() { return g_forced_threads; }

int grouped_kernel_variant() { return g_grouped_variant; }
thread_local int g_route_split = 0;
int route_split_forced() { return g_route_split; }

int device_limits(DeviceLimits* out)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error("hipGetDevice failed: %s", hipGetErrorString(err));
        return FTQ_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_lim_mu);
    DeviceLimits& l = g_lim[dev];
    if (l.device != dev) {
        int gx = 0, thr = 0, lds = 0, cus = 0;
        if (hipDeviceGetAttribute(&gx, hipDeviceAttributeMaxGridDimX, dev) != hipSuccess ||
            hipDeviceGetAttribute(&thr, hipDeviceAttributeMaxThreadsPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            set_error("hipDeviceGetAttribute failed on device %d", dev);
            return FTQ_ERR_HIP;
        }
        l.max_grid_x = gx;
        l.max_threads = thr;
        l.max_lds = lds;
        l.cu_count = cus;
        l.device = dev;
    }
    *out = l;
    return FTQ_OK;
}

int64_t stride_grid(int64_t needed, const DeviceLimits& lim, int per_cu)
{
    const int64_t cap = (int64_t)std::max(lim.cu_count, 1) * per_cu;
    return std::max<int64_t>(1, std::min(needed, std::min(cap, lim.max_grid_x)));
}

namespace {

int check_sizes(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k)
{
    if (K <= 0 || K % kQK != 0) { set_error("K must be a positive multiple of 32 (got %lld)", (long long)K); return FTQ_ERR_INVALID_ARG; }
    if (E < 1 || N < 1 || top_k < 1 || T < 0) {
        set_error("need E >= 1, N >= 1, top_k >= 1, T >= 0 (got E=%lld N=%lld top_k=%lld T=%lld)",
                  (long long)E, (long long)N, (long long)top_k, (long long)T);
        return FTQ_ERR_INVALID_ARG;
    }
    if (top_k > E) { set_error("top_k (%lld) exceeds the number of experts (%lld)", (long long)top_k, (long long)E); return FTQ_ERR_INVALID_ARG; }
    if (T > kMaxPairs / top_k) {
        set_error("T*top_k = %lld*%lld exceeds the 2^31-1 pair limit", (long long)T, (long long)top_k);
        return FTQ_ERR_UNSUPPORTED;
    }
    if (E > kMaxExperts) { set_error("E = %lld exceeds the supported %lld experts", (long long)E, (long long)kMaxExperts); return FTQ_ERR_UNSUPPORTED; }
    // every byte offset must fit int64: E*N*(K/32)*18 and T*top_k*N*4
    const int64_t nb = K / kQK;
    if (N > INT64_MAX / 64 / E / nb || (T * top_k) > INT64_MAX / 64 / N) {
        set_error("tensor sizes overflow 64-bit byte offsets");
        return FTQ_ERR_UNSUPPORTED;
    }
    return FTQ_OK;
}

int select_path(int64_t E, int64_t T, int64_t top_k)
{
    const int64_t pairs = T * top_k;
    // few pairs per expert: stream each expert's rows once and serve its pairs
    // on the vector ALUs; otherwise sorted MFMA tiles.  The crossover, measured
    // on one MI355X: about 7 pairs per expert with 8 experts (14336 x 4096
    // rows), about 4 with 128 (1408 x 2816).
    const int64_t per_expert_x2 = E <= 16 ? 14 : 8;   // twice the pairs per expert
    if (pairs <= kGemvScanMaxPairs && 2 * pairs <= per_expert_x2 * E) return FTQ_PATH_GEMV;
    return FTQ_PATH_GROUPED;
}

int64_t tile_m_for(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k)
{
    MoeArgs m{};
    m.E = E; m.N = N; m.K = K; m.T = T; m.top_k = top_k; m.wtype = FTQ_W_Q4_0;
    return grouped_tile_m(m);
}

// Workspace plan for a resolved path; `bucketed` tells whether the plan is used.
BucketPlan plan_for(int path, int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, bool* bucketed)
{
    const int64_t pairs = T * top_k;
    if (path == FTQ_PATH_GEMV && pairs <= kGemvScanMaxPairs) {
        *bucketed = false;
        return BucketPlan{};
    }
    *bucketed = true;
    const int64_t tm = path == FTQ_PATH_GROUPED ? tile_m_for(E, N, K, T, top_k) : 0;
    return make_bucket_plan(pairs, E, tm);
}

int resolve_path(int path, int64_t E, int64_t T, int64_t top_k)
{
    if (path == FTQ_PATH_AUTO) return select_path(E, T, top_k);
    if (path == FTQ_PATH_GEMV || path == FTQ_PATH_GROUPED) return path;
    return -1;
}

int check_workspace(int64_t need, const void* ws, size_t ws_bytes)
{
    if (!ws || (int64_t)ws_bytes < need) {
        set_error("workspace of %zu bytes is smaller than the %lld bytes needed", ws_bytes, (long long)need);
        return FTQ_ERR_WORKSPACE;
    }
    if (!aligned(ws, 256)) { set_error("workspace must be 256-byte aligned"); return FTQ_ERR_INVALID_ARG; }
    return FTQ_OK;
}

// kRoute: bucketing only; kMatmul: matmul only (pairs already routed); both: the full call.
enum Phase { kRoute = 1, kMatmul = 2 };

// act_per_pair: `a` holds one Q8_1 row per pair ([T*top_k][K/32]) instead of
// one per token ([T][K/32]).

int moe_common(const void* w, const void* a, const int32_t* ids, float* out, int32_t* partials,
               int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, void* ws, size_t ws_bytes,
               int path, hipStream_t stream, int phases, bool act_per_pair = false, int act = 0,
               int wtype = FTQ_W_Q4_0)
{
    clear_error();
    int st = check_sizes(E, N, K, T, top_k);
    if (st != FTQ_OK) return st;
    if (wtype != FTQ_W_Q4_0 && wtype != FTQ_W_Q4_1 && wtype != FTQ_W_Q5_0 && wtype != FTQ_W_Q5_1 && wtype != FTQ_W_Q8_0) {
        set_error("unknown weight type %d", wtype);
        return FTQ_ERR_INVALID_ARG;
    }
    if (wtype == FTQ_W_Q5_0 || wtype == FTQ_W_Q5_1) {
        // the five-bit types run on the GEMV path only
        if (path == FTQ_PATH_GROUPED) {
            set_error("weight type %d: the grouped path takes Q4_0, Q4_1 and Q8_0; use FTQ_PATH_GEMV or FTQ_PATH_AUTO", wtype);
            return FTQ_ERR_UNSUPPORTED;
        }
        if (path == FTQ_PATH_AUTO) path = FTQ_PATH_GEMV;
    }
    if (act != 0) {
        if (act != FTQ_ACT_SILU && act != FTQ_ACT_GELU_TANH) { set_error("unknown activation %d", act); return FTQ_ERR_INVALID_ARG; }
        if (N % 2 != 0) { set_error("a gated activation needs an even N (gate and up halves), got %lld", (long long)N); return FTQ_ERR_INVALID_ARG; }
    }
    const int rp = resolve_path(path, E, T, top_k);
    if (rp < 0) { set_error("unknown path %d", path); return FTQ_ERR_INVALID_ARG; }
    if (T == 0) return FTQ_OK;
    if (!ids || ((phases & kMatmul) && (!w || !a || (!out && !partials)))) {
        set_error("null pointer argument (w, a, topk_ids or the output)");
        return FTQ_ERR_INVALID_ARG;
    }
    if (!aligned(ids, 4) || ((phases & kMatmul) &&
        (!aligned(w, 2) || !aligned(a, 4) || !aligned(out ? (const void*)out : (const void*)partials, 4)))) {
        set_error("misaligned pointer (w needs 2-byte, a/topk_ids/out 4-byte alignment)");
        return FTQ_ERR_INVALID_ARG;
    }
    bool bucketed = false;
    const BucketPlan plan = plan_for(rp, E, N, K, T, top_k, &bucketed);
    if (bucketed) {
        // the workspace holds the bucket tables (both paths read the activations in place)
        st = check_workspace(plan.bytes, ws, ws_bytes);
        if (st != FTQ_OK) return st;
        if (phases & kRoute) {
            st = run_bucket(ids, E, plan, ws, stream);
            if (st != FTQ_OK) return st;
        }
    }
    if (!(phases & kMatmul)) return FTQ_OK;
    MoeArgs m{w, a, ids, out, partials, E, N, K, T, top_k, act_per_pair ? 1 : top_k, act, wtype};
    if (rp == FTQ_PATH_GEMV) return run_gemv(m, bucketed ? &plan : nullptr, ws, stream);
    return run_grouped(m, plan, ws, stream);
}

int64_t workspace_bytes(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path, bool act_per_pair)
{
    (void)act_per_pair;   // the workspace does not depend on how the activations are laid out
    clear_error();
    if (check_sizes(E, N, K, T, top_k) != FTQ_OK) return -1;
    const int rp = resolve_path(path, E, T, top_k);
    if (rp < 0) { set_error("unknown path %d", path); return -1; }
    if (T == 0) return 0;
    bool bucketed = false;
    const BucketPlan plan = plan_for(rp, E, N, K, T, top_k, &bucketed);
    if (!bucketed) return 0;
    return plan.bytes;
}

}  // namespace

int moe_q4_0_q8_1_call(const void* w, const void* a, const int32_t* ids, float* out, int64_t E, int64_t N, int64_t K,
                       int64_t T, int64_t top_k, void* ws, size_t ws_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, ids, out, nullptr, E, N, K, T, top_k, ws, ws_bytes, path, stream, kRoute | kMatmul);
}

int64_t moe_workspace_need(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path, int* status)
{
    clear_error();
    *status = check_sizes(E, N, K, T, top_k);
    if (*status != FTQ_OK) return -1;
    const int rp = resolve_path(path, E, T, top_k);
    if (rp < 0) {
        set_error("unknown path %d", path);
        *status = FTQ_ERR_INVALID_ARG;
        return -1;
    }
    if (T == 0) return 0;
    bool bucketed = false;
    const BucketPlan plan = plan_for(rp, E, N, K, T, top_k, &bucketed);
    return bucketed ? plan.bytes : 0;
}

}  // namespace ftq

using namespace ftq;

extern "C" {

int ftq_quantize_q8_1(const float* x, int64_t T, int64_t K, void* y, hipStream_t stream)
{
    clear_error();
    if (K <= 0 || K % kQK != 0 || T < 0) { set_error("need K > 0, K %% 32 == 0, T >= 0"); return FTQ_ERR_INVALID_ARG; }
    if (T > INT64_MAX / K / 4) { set_error("T*K overflows"); return FTQ_ERR_UNSUPPORTED; }
    if (T == 0) return FTQ_OK;
    if (!x || !y) { set_error("null pointer argument"); return FTQ_ERR_INVALID_ARG; }
    if (!aligned(x, 16) || !aligned(y, 4)) { set_error("x must be 16-byte and y 4-byte aligned"); return FTQ_ERR_INVALID_ARG; }
    return run_quantize_q8_1(x, T, K, y, stream);
}

int ftq_quantize_q4_0(const float* w, int64_t rows, int64_t K, void* y, hipStream_t stream)
{
    clear_error();
    if (K <= 0 || K % kQK != 0 || rows < 0) { set_error("need K > 0, K %% 32 == 0, rows >= 0"); return FTQ_ERR_INVALID_ARG; }
    if (rows > INT64_MAX / K / 4) { set_error("rows*K overflows"); return FTQ_ERR_UNSUPPORTED; }
    if (rows == 0) return FTQ_OK;
    if (!w || !y) { set_error("null pointer argument"); return FTQ_ERR_INVALID_ARG; }
    if (!aligned(w, 16) || !aligned(y, 2)) { set_error("w must be 16-byte and y 2-byte aligned"); return FTQ_ERR_INVALID_ARG; }
    return run_quantize_q4_0(w, rows, K, y, stream);
}

int ftq_moe_select_path(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k)
{
    clear_error();
    int st = check_sizes(E, N, K, T, top_k);
    if (st != FTQ_OK) return -st;
    return select_path(E, T, top_k);
}


int64_t ftq_moe_workspace_bytes(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path)
{
    return workspace_bytes(E, N, K, T, top_k, path, false);
}

int64_t ftq_moe_pairs_workspace_bytes(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path)
{
    return workspace_bytes(E, N, K, T, top_k, path, true);
}

int ftq_moe_q4_0_q8_1(const void* w, const void* a, const int32_t* topk_ids, float* out, int64_t E,
                      int64_t N, int64_t K, int64_t T, int64_t top_k, void* workspace,
                      size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kRoute | kMatmul);
}

int ftq_moe_route(const int32_t* topk_ids, int64_t E, int64_t T, int64_t top_k, void* workspace,
                  size_t workspace_bytes, int path, hipStream_t stream)
{
    // N and K do not enter the routing; any valid values pass the size checks
    return moe_common(nullptr, nullptr, topk_ids, nullptr, nullptr, E, 1, kQK, T, top_k, workspace,
                      workspace_bytes, path, stream, kRoute);
}

int ftq_moe_q4_0_q8_1_routed(const void* w, const void* a, const int32_t* topk_ids, float* out, int64_t E,
                             int64_t N, int64_t K, int64_t T, int64_t top_k, void* workspace,
                             size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kMatmul);
}

int ftq_moe_q4_0_q8_1_partials(const void* w, const void* a, const int32_t* topk_ids, int32_t* partials,
                               int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                               void* workspace, size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, nullptr, partials, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kRoute | kMatmul);
}

int ftq_moe_q4_0_q8_1_pairs(const void* w, const void* a_pairs, const int32_t* topk_ids, float* out, int64_t E,
                            int64_t N, int64_t K, int64_t T, int64_t top_k, void* workspace,
                            size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a_pairs, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path,
                      stream, kRoute | kMatmul, true);
}

int ftq_moe_q4_0_q8_1_pairs_routed(const void* w, const void* a_pairs, const int32_t* topk_ids, float* out,
                                   int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, void* workspace,
                                   size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a_pairs, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path,
                      stream, kMatmul, true);
}

int ftq_moe_q4_0_q8_1_pairs_partials(const void* w, const void* a_pairs, const int32_t* topk_ids,
                                     int32_t* partials, int64_t E, int64_t N, int64_t K, int64_t T,
                                     int64_t top_k, void* workspace, size_t workspace_bytes, int path,
                                     hipStream_t stream)
{
    return moe_common(w, a_pairs, topk_ids, nullptr, partials, E, N, K, T, top_k, workspace, workspace_bytes, path,
                      stream, kRoute | kMatmul, true);
}

int ftq_moe_combine_topk(const float* y, const float* gates, float* out, int64_t T, int64_t top_k, int64_t N,
                         hipStream_t stream)
{
    clear_error();
    if (T < 0 || top_k < 1 || N < 1) {
        set_error("need T >= 0, top_k >= 1, N >= 1 (got T=%lld top_k=%lld N=%lld)", (long long)T, (long long)top_k,
                  (long long)N);
        return FTQ_ERR_INVALID_ARG;
    }
    if (T > INT64_MAX / 8 / top_k / N) { set_error("T*top_k*N overflows 64-bit byte offsets"); return FTQ_ERR_UNSUPPORTED; }
    if (T == 0) return FTQ_OK;
    if (!y || !gates || !out) { set_error("null pointer argument (y, gates or out)"); return FTQ_ERR_INVALID_ARG; }
    if (!aligned(y, 4) || !aligned(gates, 4) || !aligned(out, 4)) {
        set_error("misaligned pointer (y, gates and out need 4-byte alignment)");
        return FTQ_ERR_INVALID_ARG;
    }
    return run_combine_topk(y, gates, out, T, top_k, N, stream);
}

int ftq_moe_q4_0_q8_1_act(const void* w, const void* a, const int32_t* topk_ids, float* out, int64_t E,
                          int64_t N, int64_t K, int64_t T, int64_t top_k, int act, void* workspace,
                          size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kRoute | kMatmul, false, act);
}

int ftq_moe_q4_0_q8_1_act_routed(const void* w, const void* a, const int32_t* topk_ids, float* out, int64_t E,
                                 int64_t N, int64_t K, int64_t T, int64_t top_k, int act, void* workspace,
                                 size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kMatmul, false, act);
}

int ftq_moe_gguf_q8_1(const void* w, int wtype, const void* a, const int32_t* topk_ids, float* out, int64_t E,
                      int64_t N, int64_t K, int64_t T, int64_t top_k, int act_per_pair, void* workspace,
                      size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, out, nullptr, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kRoute | kMatmul, act_per_pair != 0, 0, wtype);
}

int ftq_moe_gguf_q8_1_partials(const void* w, int wtype, const void* a, const int32_t* topk_ids, int32_t* partials,
                               int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int act_per_pair,
                               void* workspace, size_t workspace_bytes, int path, hipStream_t stream)
{
    return moe_common(w, a, topk_ids, nullptr, partials, E, N, K, T, top_k, workspace, workspace_bytes, path, stream,
                      kRoute | kMatmul, act_per_pair != 0, 0, wtype);
}

const char* ftq_last_error(void) { return g_error.c_str(); }

const char* ftq_version(void) { return "ftq 0.1.0 gfx950"; }

void ftq_debug_force_block_threads(int threads) { g_forced_threads = threads > 0 ? threads : 0; }

void ftq_debug_route_kernels(int split) { g_route_split = split ? 1 : 0; }

int ftq_debug_grouped_kernel(int variant)
{
    clear_error();
    if (variant < kGroupedI8 || variant > kGroupedF16Ws) {
        set_error("grouped kernel variant %d: expected 0 (int8), 1 (fp16) or 2 (fp16, warp-specialised)", variant);
        return FTQ_ERR_INVALID_ARG;
    }
    g_grouped_variant = variant;
    return FTQ_OK;
}

int ftq_debug_gemv_plan(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int wtype, int act, int64_t* seg,
                        int64_t* pairs_per_pass, int64_t* wg_per_cu)
{
    clear_error();
    int st = check_sizes(E, N, K, T, top_k);
    if (st != FTQ_OK) return st;
    if (!seg || !pairs_per_pass || !wg_per_cu) { set_error("null output pointer"); return FTQ_ERR_INVALID_ARG; }
    MoeArgs m{};
    m.E = E; m.N = N; m.K = K; m.T = T; m.top_k = top_k; m.act = act; m.wtype = wtype;
    const GemvPlan g = plan_gemv(m, T * top_k > kGemvScanMaxPairs);
    if (!g.fits) { set_error("a fused activation row of K = %lld does not fit on chip", (long long)K); return FTQ_ERR_UNSUPPORTED; }
    *seg = g.seg;
    *pairs_per_pass = g.pc_cap;
    *wg_per_cu = g.per_cu;
    return FTQ_OK;
}

}  // extern "C"
