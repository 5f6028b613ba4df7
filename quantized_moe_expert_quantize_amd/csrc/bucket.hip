// Bucketing of the flat (token, top-k) pairs by routed expert, for the
// expert-sorted paths: per-chunk expert histogram -> exclusive scan into
// per-expert segment offsets (the "expert_offsets" of "Current Bug:
// CuTeDSLMoERunner", Bug 4, kept here WITH the leading 0 and the total) and a
// per-expert tile count scan -> stable scatter of pair ids into their expert's
// segment.  Ids outside [0, E) go to one extra bucket E, whose rows the matmul
// writes as zeros (that page's Bug 8: non-local experts are masked).
//
// Every pass is deterministic: counts do not depend on the order of LDS
// atomics, and the scatter orders each chunk with a bitonic sort on the unique
// key (bucket, position), so a bucket's segment lists its pairs in ascending
// pair order.  Nothing is read back to the host, so the whole sequence can be
// captured in a HIP graph ("Cudagraph Constraints" on the same page).
#include "ftq_internal.h"

namespace ftq {
namespace {

constexpr int kCountThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kSortThreads = 256;
constexpr uint32_t kPadKey = 0xffffffffu;
constexpr int kPosBits = 10;   // kBucketChunk == 1 << kPosBits
static_assert(kBucketChunk == (1 << kPosBits), "chunk size must match the key layout");

__device__ __forceinline__ int bucket_of(int32_t id, int32_t E) { return (id >= 0 && id < E) ? id : E; }

// Pass 1: counts[c][b] = number of pairs of chunk c in bucket b.
__global__ __launch_bounds__(kCountThreads) void bucket_count_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int32_t E, int32_t nbuckets,
    int32_t* __restrict__ counts)
{
    extern __shared__ int32_t hist[];
    const int64_t c = blockIdx.x;
    for (int b = threadIdx.x; b < nbuckets; b += kCountThreads) hist[b] = 0;
    __syncthreads();
    const int64_t base = c * kBucketChunk;
    for (int i = threadIdx.x; i < kBucketChunk; i += kCountThreads) {
        const int64_t p = base + i;
        if (p < pairs) atomicAdd(&hist[bucket_of(ids[p], E)], 1);
    }
    __syncthreads();
    int32_t* row = counts + c * (int64_t)nbuckets;
    for (int b = threadIdx.x; b < nbuckets; b += kCountThreads) row[b] = hist[b];
}

// Exclusive block-wide scan of v[0..n) in LDS (n <= kMaxScan), result in place;
// returns the total.  All threads of the block must call it.
__device__ int32_t block_exclusive_scan(int32_t* v, int n, int32_t* warp_tmp)
{
    // Each thread owns a contiguous run of ceil(n / blockDim) entries.
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int beg = min(n, (int)threadIdx.x * per), end = min(n, beg + per);
    int32_t local = 0;
    for (int i = beg; i < end; ++i) local += v[i];
    // inclusive scan of `local` across the block: wave scan, then over waves
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t x = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) warp_tmp[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;
        for (int w = 0; w < kScanThreads / 64; ++w) { int32_t t = warp_tmp[w]; warp_tmp[w] = run; run += t; }
        warp_tmp[kScanThreads / 64] = run;
    }
    __syncthreads();
    int32_t run = warp_tmp[wave] + x - local;   // exclusive prefix of this thread's run
    for (int i = beg; i < end; ++i) { int32_t t = v[i]; v[i] = run; run += t; }
    const int32_t total = warp_tmp[kScanThreads / 64];
    __syncthreads();
    return total;
}

// Pass 2 (one block): bucket offsets, per-chunk bases (in place over counts),
// and the per-bucket first-tile table.
__global__ __launch_bounds__(kScanThreads) void bucket_scan_kernel(
    int32_t* __restrict__ counts, int64_t nchunks, int32_t nbuckets, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tiles)
{
    extern __shared__ int32_t lds[];
    int32_t* tot = lds;                       // [nbuckets]
    int32_t* ntile = lds + nbuckets;          // [nbuckets]
    __shared__ int32_t warp_tmp[kScanThreads / 64 + 1];
    for (int b = threadIdx.x; b < nbuckets; b += kScanThreads) {
        int32_t s = 0;
        for (int64_t c = 0; c < nchunks; ++c) s += counts[c * nbuckets + b];
        tot[b] = s;
        ntile[b] = tile_m > 0 ? (s + tile_m - 1) / tile_m : 0;
    }
    __syncthreads();
    // tot -> exclusive offsets
    const int32_t total = block_exclusive_scan(tot, nbuckets, warp_tmp);
    const int32_t total_tiles = block_exclusive_scan(ntile, nbuckets, warp_tmp);
    for (int b = threadIdx.x; b < nbuckets; b += kScanThreads) {
        offsets[b] = tot[b];
        tiles[b] = ntile[b];
        int32_t run = tot[b];
        for (int64_t c = 0; c < nchunks; ++c) {
            int32_t n = counts[c * nbuckets + b];
            counts[c * nbuckets + b] = run;
            run += n;
        }
    }
    if (threadIdx.x == 0) {
        offsets[nbuckets] = total;
        tiles[nbuckets] = total_tiles;
    }
}

// Pass 3: sort each chunk by (bucket, position) and scatter pair ids to
// bases[c][b] + (rank within the chunk's run of bucket b).
__global__ __launch_bounds__(kSortThreads) void bucket_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int32_t E, int32_t nbuckets,
    const int32_t* __restrict__ bases, int32_t* __restrict__ sorted)
{
    __shared__ uint32_t key[kBucketChunk];
    const int64_t c = blockIdx.x;
    const int64_t base = c * kBucketChunk;
    for (int i = threadIdx.x; i < kBucketChunk; i += kSortThreads) {
        const int64_t p = base + i;
        key[i] = (p < pairs) ? (((uint32_t)bucket_of(ids[p], E) << kPosBits) | (uint32_t)i) : kPadKey;
    }
    __syncthreads();
    // bitonic sort, ascending; keys are unique (the position is part of the key)
    for (int k = 2; k <= kBucketChunk; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < kBucketChunk; i += kSortThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint32_t a = key[i], b = key[ixj];
                    const bool ascending = (i & k) == 0;
                    if ((a > b) == ascending) { key[i] = b; key[ixj] = a; }
                }
            }
            __syncthreads();
        }
    }
    const int32_t* crow = bases + c * (int64_t)nbuckets;
    for (int s = threadIdx.x; s < kBucketChunk; s += kSortThreads) {
        const uint32_t k = key[s];
        if (k == kPadKey) continue;
        const uint32_t b = k >> kPosBits;
        // first sorted slot holding bucket b (lower bound of b << kPosBits)
        int lo = 0, hi = s;
        const uint32_t first = b << kPosBits;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (key[mid] < first) lo = mid + 1; else hi = mid;
        }
        sorted[crow[b] + (s - lo)] = (int32_t)(base + (k & ((1u << kPosBits) - 1)));
    }
}

}  // namespace

BucketPlan make_bucket_plan(int64_t pairs, int64_t E, int64_t tile_m)
{
    BucketPlan p;
    p.pairs = pairs;
    p.buckets = E + 1;
    p.chunks = (pairs + kBucketChunk - 1) / kBucketChunk;
    p.tile_m = tile_m;
    auto align = [](int64_t v) { return (v + 255) / 256 * 256; };
    int64_t off = 0;
    p.off_counts = off;  off = align(off + 4 * p.chunks * p.buckets);
    p.off_offsets = off; off = align(off + 4 * (p.buckets + 1));
    p.off_tiles = off;   off = align(off + 4 * (p.buckets + 1));
    p.off_sorted = off;  off = align(off + 4 * pairs);
    p.bytes = off;
    return p;
}

int run_bucket(const int32_t* ids, int64_t E, const BucketPlan& plan, void* ws, hipStream_t s)
{
    if (plan.pairs == 0) return FTQ_OK;
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(base + plan.off_counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + plan.off_offsets);
    int32_t* tiles = reinterpret_cast<int32_t*>(base + plan.off_tiles);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + plan.off_sorted);
    const int32_t nb = (int32_t)plan.buckets;
    int st = launch("bucket_count_kernel", bucket_count_kernel, plan.chunks, kCountThreads,
                    sizeof(int32_t) * nb, s, ids, plan.pairs, (int32_t)E, nb, counts);
    if (st != FTQ_OK) return st;
    st = launch("bucket_scan_kernel", bucket_scan_kernel, 1, kScanThreads, 2 * sizeof(int32_t) * nb, s,
                counts, plan.chunks, nb, (int32_t)plan.tile_m, offsets, tiles);
    if (st != FTQ_OK) return st;
    return launch("bucket_scatter_kernel", bucket_scatter_kernel, plan.chunks, kSortThreads, 0, s, ids,
                  plan.pairs, (int32_t)E, nb, static_cast<const int32_t*>(counts), sorted);
}

}  // namespace ftq
