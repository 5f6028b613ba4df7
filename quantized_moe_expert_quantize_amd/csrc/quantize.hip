// Quantisers: fp32 activations -> Q8_1 blocks (the step that runs right before
// the MoE GEMV; FreeToken PR #185, Fix, "quantize_row_q8_1_cuda"), and fp32
// weights -> Q4_0 blocks (weight preparation).
//
// Both are HBM-streaming kernels.  Every loop walks a 64-bit flat block index
// with a grid stride, so any number of rows runs in one launch (the same
// concern as the 65535 grid limit in FreeToken PR #185, Problem).
#include "ftq_internal.h"

namespace ftq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> fp16 bits, round to nearest even.  The empty asm pins `f` as an
// fp32 register value: without it the backend folds a preceding fp32 multiply
// and this conversion into one v_fma_mix (a single rounding), whereas the
// format rounds the product to fp32 first and then to fp16.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    __asm__ volatile("" : "+v"(f));
    _Float16 h = (_Float16)f;   // v_cvt_f16_f32
    return __builtin_bit_cast(uint16_t, h);
}

// Q8_1: four lanes per 32-value block, eight values per lane (two float4).
constexpr int kQ8Threads = 256;
constexpr int kQ8BlocksPerGroup = kQ8Threads / 4;

__global__ __launch_bounds__(kQ8Threads) void quantize_q8_1_kernel(
    const float* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ y)
{
    const int sub = threadIdx.x & 3;
    const int64_t stride = (int64_t)gridDim.x * kQ8BlocksPerGroup;
    for (int64_t blk = (int64_t)blockIdx.x * kQ8BlocksPerGroup + (threadIdx.x >> 2); blk < nblocks;
         blk += stride) {
        // x is [T][K] with K % 32 == 0, so block (t, b) starts at float blk*32.
        const f32x4* src = reinterpret_cast<const f32x4*>(x + blk * kQK + sub * 8);
        const f32x4 v0 = __builtin_nontemporal_load(src);
        const f32x4 v1 = __builtin_nontemporal_load(src + 1);
        float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const float d = amax / 127.0f;   // correctly rounded fp32 division
        int q[8];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            q[i] = (amax == 0.0f) ? 0 : (int)roundf(v[i] / d);   // half away from zero
            sum += q[i];
        }
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        const float s = d * (float)sum;
        uint32_t lo = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                      ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
        uint32_t hi = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) |
                      ((uint32_t)(q[6] & 0xff) << 16) | ((uint32_t)(q[7] & 0xff) << 24);
        uint32_t* dst = reinterpret_cast<uint32_t*>(y + blk * kQ8Bytes);   // 36-byte blocks: 4-aligned
        dst[1 + 2 * sub] = lo;
        dst[2 + 2 * sub] = hi;
        if (sub == 0) dst[0] = (uint32_t)f32_to_f16_bits(d) | ((uint32_t)f32_to_f16_bits(s) << 16);
    }
}

// Q4_0: one lane per block (weight preparation, not on the timed path).
constexpr int kQ4Threads = 256;

__global__ __launch_bounds__(kQ4Threads) void quantize_q4_0_kernel(
    const float* __restrict__ w, int64_t nblocks, uint8_t* __restrict__ y)
{
    const int64_t stride = (int64_t)gridDim.x * kQ4Threads;
    for (int64_t blk = (int64_t)blockIdx.x * kQ4Threads + threadIdx.x; blk < nblocks; blk += stride) {
        const float4* src = reinterpret_cast<const float4*>(w + blk * kQK);
        float v[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 f = src[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
        float m = 0.0f, amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (fabsf(v[i]) > amax) { amax = fabsf(v[i]); m = v[i]; }   // first index on ties
        }
        const float d = m / -8.0f;
        uint16_t* dst = reinterpret_cast<uint16_t*>(y + blk * kQ4Bytes);   // 18-byte blocks: 2-aligned
        dst[0] = f32_to_f16_bits(d);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int qa[2], qb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e0 = 2 * i + h, e1 = e0 + 16;
                int c0 = 8, c1 = 8;
                if (d != 0.0f) {
                    c0 = min(15, max(0, (int)roundf(v[e0] / d) + 8));
                    c1 = min(15, max(0, (int)roundf(v[e1] / d) + 8));
                }
                qa[h] = c0;
                qb[h] = c1;
            }
            const uint32_t b0 = (uint32_t)(qa[0] | (qb[0] << 4));
            const uint32_t b1 = (uint32_t)(qa[1] | (qb[1] << 4));
            dst[1 + i] = (uint16_t)(b0 | (b1 << 8));
        }
    }
}

}  // namespace

int run_quantize_q8_1(const float* x, int64_t T, int64_t K, void* y, hipStream_t s)
{
    const int64_t nblocks = T * (K / kQK);
    if (nblocks == 0) return FTQ_OK;
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    const int64_t groups = (nblocks + kQ8BlocksPerGroup - 1) / kQ8BlocksPerGroup;
    return launch("quantize_q8_1_kernel", quantize_q8_1_kernel, stride_grid(groups, lim), kQ8Threads, 0,
                  s, x, nblocks, static_cast<uint8_t*>(y));
}

int run_quantize_q4_0(const float* w, int64_t rows, int64_t K, void* y, hipStream_t s)
{
    const int64_t nblocks = rows * (K / kQK);
    if (nblocks == 0) return FTQ_OK;
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    const int64_t groups = (nblocks + kQ4Threads - 1) / kQ4Threads;
    return launch("quantize_q4_0_kernel", quantize_q4_0_kernel, stride_grid(groups, lim), kQ4Threads, 0,
                  s, w, nblocks, static_cast<uint8_t*>(y));
}

}  // namespace ftq
