// ftq_moe_q4_0_q8_1 for callers that cannot allocate device memory (code
// under graph capture, tight serving loops, harnesses that forbid it): the
// workspace is a fixed-size array that the library holds on every device it
// runs on, so the caller passes only inputs and outputs.
//
// `scratch` is a device variable: in host code its name stands for a host-side
// shadow, not for device memory.  Its device address is taken once per device
// with hipGetSymbolAddress (with that device current) and only that address
// is handed to kernels.  The bucketing kernels write every workspace entry
// before reading it, so nothing has to be cleared between calls.  All calls on
// one device share the array: calls that overlap on one device (other streams,
// other threads) race on it.
#include <mutex>

#include "ftq_internal.h"

namespace ftq {
namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;   // 4 MiB per device
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices] = {};

// Device address of this device's `scratch`, looked up on first use.
int scratch_address(void** out)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        set_error("hipGetDevice failed: %s", hipGetErrorString(err));
        return FTQ_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p) {
            set_error("hipGetSymbolAddress of the scratch array failed on device %d: %s", dev, hipGetErrorString(err));
            return FTQ_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FTQ_OK;
}

}  // namespace
}  // namespace ftq

using namespace ftq;

extern "C" int ftq_moe_q4_0_q8_1_noalloc(const void* w, const void* a, const int32_t* topk_ids, float* out, int64_t E,
                                         int64_t N, int64_t K, int64_t T, int64_t top_k, int path, hipStream_t stream)
{
    int st = FTQ_OK;
    const int64_t need = moe_workspace_need(E, N, K, T, top_k, path, &st);
    if (st != FTQ_OK) return st;
    if (need > (int64_t)kScratchBytes) {
        set_error("this call needs %lld bytes of workspace, more than the %zu bytes of fixed scratch per device; "
                  "use ftq_moe_q4_0_q8_1 with a caller-provided workspace",
                  (long long)need, kScratchBytes);
        return FTQ_ERR_UNSUPPORTED;
    }
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != FTQ_OK) return st;
    }
    return moe_q4_0_q8_1_call(w, a, topk_ids, out, E, N, K, T, top_k, ws, need > 0 ? kScratchBytes : 0, path, stream);
}
