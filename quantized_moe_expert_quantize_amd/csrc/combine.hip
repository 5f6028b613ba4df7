// Top-k weighted combine of the expert outputs of a token's pairs: the step
// after the down projection of an expert FFN (the per-pair activation layout
// of "Current Bug: CuTeDSLMoERunner", Bug 6, and its L2 output).
//
//   out[t][n] = sum_{j < k} gates[t][j] * y[t*k + j][n]
//
// evaluated in fp32 as acc = fma(gates[t][j], y[t*k+j][n], acc) for j = 0, 1,
// ..., k-1 from acc = 0: a fixed order, so the result does not depend on the
// batch or the launch.  Rows of masked pairs hold zeros (the matmul writes
// them) and add nothing.  The kernel streams y once: HBM bound, with four
// consecutive columns per lane (16-byte loads and stores) when N % 4 == 0 and
// the buffers are 16-byte aligned.
#include "ftq_internal.h"

namespace ftq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int VEC>
__global__ __launch_bounds__(kThreads) void combine_topk_kernel(const float* __restrict__ y,
                                                                const float* __restrict__ gates,
                                                                float* __restrict__ out, int64_t T, int64_t k,
                                                                int64_t N)
{
    const int64_t nv = N / VEC;                       // column groups per row
    const int64_t total = T * nv;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
        const int64_t t = i / nv, c = (i - t * nv) * VEC;
        if constexpr (VEC == 4) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int64_t j = 0; j < k; ++j) {
                const float g = gates[t * k + j];
                const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (t * k + j) * N + c));
                acc.x = __builtin_fmaf(g, v.x, acc.x);
                acc.y = __builtin_fmaf(g, v.y, acc.y);
                acc.z = __builtin_fmaf(g, v.z, acc.z);
                acc.w = __builtin_fmaf(g, v.w, acc.w);
            }
            *reinterpret_cast<f32x4*>(out + t * N + c) = acc;
        } else {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; ++j) acc = __builtin_fmaf(gates[t * k + j], y[(t * k + j) * N + c], acc);
            out[t * N + c] = acc;
        }
    }
}

}  // namespace

int run_combine_topk(const float* y, const float* gates, float* out, int64_t T, int64_t top_k, int64_t N,
                     hipStream_t s)
{
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    const bool v4 = N % 4 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    const int64_t items = T * (v4 ? N / 4 : N);
    const int64_t grid = stride_grid((items + kThreads - 1) / kThreads, lim);
    if (v4) return launch("combine_topk_kernel<4>", combine_topk_kernel<4>, grid, kThreads, 0, s, y, gates, out, T, top_k, N);
    return launch("combine_topk_kernel<1>", combine_topk_kernel<1>, grid, kThreads, 0, s, y, gates, out, T, top_k, N);
}

}  // namespace ftq
