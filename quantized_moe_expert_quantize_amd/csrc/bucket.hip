// Bucketing of the flat (token, top-k) pairs by routed expert, for the
// expert-sorted paths: per-chunk expert histogram -> one exclusive scan that
// yields the per-expert segment offsets (the "expert_offsets" of "Current
// Bug: CuTeDSLMoERunner", Bug 4, kept here WITH the leading 0 and the total),
// every chunk's base inside its expert's segment, and the per-expert tile
// table -> stable scatter of pair ids into their expert's segment.  Ids
// outside [0, E) go to one extra bucket E, whose rows the matmul writes as
// zeros (that page's Bug 8: non-local experts are masked).
//
// The counts are stored bucket-major, counts[b][c] for bucket b and chunk c,
// so a single flat exclusive scan over them gives, at [b][c], the sorted
// position of chunk c's first pair of bucket b: the pairs of lower buckets,
// then those of bucket b in earlier chunks.
//
// Every pass is deterministic: counts do not depend on the order of LDS
// atomics, and the scatter walks each chunk in pair order (one wave per chunk,
// 64 pairs per step, ranks within a step from ballots), so a bucket's segment
// lists its pairs in ascending pair order.  Nothing is read back to the host,
// so the whole sequence can be captured in a HIP graph ("Cudagraph
// Constraints" on the same page).
#include "ftq_internal.h"

namespace ftq {
namespace {

constexpr int kCountThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;                  // elements per thread and pass of the flat scan
constexpr int kScatterWaves = 4;             // chunks per scatter workgroup (one wave each)
constexpr int kKeyBits = 12;                 // bucket ids < 4096

__device__ __forceinline__ int bucket_of(int32_t id, int32_t E) { return (id >= 0 && id < E) ? id : E; }

// Pass 1: counts[b][c] = number of pairs of chunk c in bucket b.
__global__ __launch_bounds__(kCountThreads) void bucket_count_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int32_t E, int32_t nbuckets, int64_t nchunks,
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
    for (int b = threadIdx.x; b < nbuckets; b += kCountThreads) counts[(int64_t)b * nchunks + c] = hist[b];
}

// Exclusive prefix of v over the threads of the block, in thread order, plus
// `carry`; carry becomes carry + the block's total.  wsum: kScanWaves + 1
// ints of LDS.  Every thread must call it (three barriers).
constexpr int kScanWaves = kScanThreads / 64;
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t& carry, int32_t* wsum)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {   // scan of the wave totals, in one wave
        const int32_t t = lane < kScanWaves ? wsum[lane] : 0;
        int32_t u = t;
#pragma unroll
        for (int o = 1; o < kScanWaves; o <<= 1) {
            const int32_t y = __shfl_up(u, o);
            if (lane >= o) u += y;
        }
        if (lane < kScanWaves) wsum[lane] = u - t;
        if (lane == kScanWaves - 1) wsum[kScanWaves] = u;
    }
    __syncthreads();
    const int32_t r = carry + wsum[wave] + x - v;
    const int32_t total = wsum[kScanWaves];
    __syncthreads();   // wsum is rewritten by the next call
    carry += total;
    return r;
}

// The bucket offsets (from off_lds[0..nbuckets], in LDS), the exclusive scan of
// the per-bucket tile counts and one descriptor per tile; tiles_lds: nbuckets + 1
// ints of LDS.  Every thread of the block must call it.
__device__ void write_tables(int32_t nbuckets, int32_t tile_m, const int32_t* off_lds, int32_t* tiles_lds,
                             int32_t* wsum, int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                             int4* __restrict__ tdesc)
{
    for (int b = threadIdx.x; b <= nbuckets; b += kScanThreads) offsets[b] = off_lds[b];
    int32_t tcarry = 0;
    for (int b0 = 0; b0 < nbuckets; b0 += kScanThreads) {
        const int b = b0 + (int)threadIdx.x;
        const int32_t n = b < nbuckets ? off_lds[b + 1] - off_lds[b] : 0;
        const int32_t t = tile_m > 0 ? (int32_t)(((uint32_t)n + (uint32_t)tile_m - 1u) / (uint32_t)tile_m) : 0;
        const int32_t r = block_exclusive_scan(t, tcarry, wsum);
        if (b < nbuckets) {
            tiles[b] = r;
            tiles_lds[b] = r;
        }
    }
    if (threadIdx.x == 0) {
        tiles[nbuckets] = tcarry;
        tiles_lds[nbuckets] = tcarry;
    }
    if (tile_m <= 0) return;
    __syncthreads();
    // One descriptor per tile {bucket, first slot, rows, 0}, so that the matmul
    // finds a tile's expert and pairs with one load instead of a search.
    for (int32_t mt = threadIdx.x; mt < tcarry; mt += kScanThreads) {
        int lo = 0, hi = nbuckets;   // the last bucket b with tiles[b] <= mt
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tiles_lds[mid] <= mt) lo = mid; else hi = mid;
        }
        const int32_t slot0 = off_lds[lo] + (mt - tiles_lds[lo]) * tile_m;
        tdesc[mt] = int4{lo, slot0, min(tile_m, off_lds[lo + 1] - slot0), 0};
    }
}

// Pass 2 (one block): flat exclusive scan of counts[nbuckets][nchunks] in
// place, the bucket offsets (offsets[b] = scanned[b][0], offsets[nbuckets] =
// pairs) and the exclusive scan of per-bucket tile counts.
__global__ __launch_bounds__(kScanThreads) void bucket_scan_kernel(
    int32_t* __restrict__ counts, int64_t nchunks, int32_t nbuckets, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tiles, int4* __restrict__ tdesc)
{
    extern __shared__ int32_t off_lds[];          // [nbuckets + 1] bucket offsets, then [nbuckets + 1] tile offsets
    int32_t* tiles_lds = off_lds + nbuckets + 1;
    __shared__ int32_t wsum[kScanWaves + 1];
    const int64_t len = (int64_t)nbuckets * nchunks;
    int32_t carry = 0;
    for (int64_t base = 0; base < len; base += (int64_t)kScanThreads * kScanPer) {
        const int64_t i0 = base + (int64_t)threadIdx.x * kScanPer;
        int32_t v[kScanPer];
        int32_t local = 0;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            v[k] = i0 + k < len ? counts[i0 + k] : 0;
            local += v[k];
        }
        int32_t run = block_exclusive_scan(local, carry, wsum);
        // bucket and chunk of element i0, then stepped along (one division per pass)
        int64_t bk = i0 / nchunks, ch = i0 - bk * nchunks;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            if (i0 + k < len) {
                counts[i0 + k] = run;
                if (ch == 0) off_lds[bk] = run;   // first chunk of bucket bk
            }
            run += v[k];
            if (++ch == nchunks) {
                ch = 0;
                ++bk;
            }
        }
    }
    if (threadIdx.x == 0) off_lds[nbuckets] = carry;
    __syncthreads();
    write_tables(nbuckets, tile_m, off_lds, tiles_lds, wsum, offsets, tiles, tdesc);
}

// Lanes of a wave share the per-bucket counters in LDS; the hardware keeps a
// wave's LDS accesses in order and the fence keeps the compiler from moving
// one lane's access across another lane's.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Pass 3: one wave per chunk walks its pairs in order, 64 at a time.  A pair's
// slot is bases[b][c] + (pairs of bucket b earlier in the chunk): the count
// from earlier steps (an LDS counter per bucket) plus the lanes below it in
// this step with the same bucket (found with one ballot per key bit).  The
// chunk's ids are loaded up front and its bases staged in LDS, so the walk
// itself waits on no global memory.
constexpr int kScatterSteps = kBucketChunk / 64;
static_assert(kBucketChunk % 64 == 0, "whole steps per chunk");

__global__ __launch_bounds__(64 * kScatterWaves) void bucket_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int32_t E, int32_t nbuckets, int64_t nchunks,
    const int32_t* __restrict__ bases, int32_t* __restrict__ sorted)
{
    extern __shared__ int32_t lds_all[];         // [kScatterWaves][2][nbuckets]: counters, chunk bases
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * kScatterWaves + wave;
    if (c >= nchunks) return;                    // whole waves only: no barrier follows
    int32_t* seen = lds_all + (int64_t)wave * 2 * nbuckets;
    int32_t* cbase = seen + nbuckets;
    const int64_t base = c * kBucketChunk;
    int32_t idv[kScatterSteps];
#pragma unroll
    for (int st = 0; st < kScatterSteps; ++st) {
        const int64_t p = base + st * 64 + lane;
        idv[st] = p < pairs ? ids[p] : 0;
    }
    for (int b = lane; b < nbuckets; b += 64) {
        seen[b] = 0;
        cbase[b] = bases[(int64_t)b * nchunks + c];
    }
    wave_lds_fence();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int st = 0; st < kScatterSteps; ++st) {
        const int64_t p = base + st * 64 + lane;
        const bool live = p < pairs;
        const int32_t b = live ? bucket_of(idv[st], E) : -1;
        // lanes holding the same bucket: agree on every key bit (and are live)
        uint64_t same = __ballot(live);
#pragma unroll
        for (int k = 0; k < kKeyBits; ++k) {
            const uint64_t ones = __ballot(live && ((b >> k) & 1));
            same &= ((b >> k) & 1) ? ones : ~ones;
        }
        if (live) {
            const int rank = __popcll(same & below);
            const int32_t prev = seen[b];
            sorted[cbase[b] + prev + rank] = (int32_t)p;
            wave_lds_fence();   // every lane has read seen[] before the leaders update it
            if (rank == 0) seen[b] = prev + __popcll(same);
        }
        wave_lds_fence();
    }
}

// All three passes in one workgroup, for batches of at most kSmallChunks
// chunks whose counts fit in LDS: the same bucket-major counts, the same flat
// scan and the same in-order scatter, so the same tables bit for bit, without
// the two kernel boundaries (and their launch and memory round trips) between
// the passes.  Wave w counts and scatters chunk w, whose ids it keeps in
// registers; the scanned counts in LDS serve as the scatter's running bases.
// Up to 8 chunks (8192 pairs) it measures 3-4 us faster than the three
// kernels (10-15 us); from about 12 chunks on, the serial walk of each wave's
// chunk makes it slower.
constexpr int kSmallChunks = 8;
constexpr int kSmallCounts = kScanThreads * kScanPer;   // buckets x chunks: one scan pass
constexpr int kSmallBuckets = 2048;
constexpr int kSmallSteps = kBucketChunk / 64;

__global__ __launch_bounds__(kScanThreads) void bucket_small_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int32_t E, int32_t nbuckets, int32_t nchunks, int32_t tile_m,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tiles, int32_t* __restrict__ sorted,
    int4* __restrict__ tdesc)
{
    // [nbuckets][nchunks] counts (then bases), [nbuckets + 1] offsets, [nbuckets + 1] tile offsets
    extern __shared__ int32_t lds_small[];
    int32_t* cnt = lds_small;
    int32_t* off_lds = cnt + nbuckets * nchunks;
    int32_t* tiles_lds = off_lds + nbuckets + 1;
    __shared__ int32_t wsum[kScanWaves + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int len = nbuckets * nchunks;
    for (int i = threadIdx.x; i < len; i += kScanThreads) cnt[i] = 0;
    __syncthreads();
    const bool mine = wave < nchunks;
    const int64_t base = (int64_t)wave * kBucketChunk;
    int32_t idv[kSmallSteps];
#pragma unroll
    for (int st = 0; st < kSmallSteps; ++st) {
        const int64_t p = base + st * 64 + lane;
        idv[st] = (mine && p < pairs) ? ids[p] : 0;
    }
    if (mine) {
#pragma unroll
        for (int st = 0; st < kSmallSteps; ++st) {
            const int64_t p = base + st * 64 + lane;
            if (p < pairs) atomicAdd(&cnt[bucket_of(idv[st], E) * nchunks + wave], 1);
        }
    }
    __syncthreads();
    // flat exclusive scan of the counts in place (len <= kSmallCounts: one pass)
    int32_t carry = 0;
    {
        const int i0 = threadIdx.x * kScanPer;
        int32_t v[kScanPer];
        int32_t local = 0;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            v[k] = i0 + k < len ? cnt[i0 + k] : 0;
            local += v[k];
        }
        int32_t run = block_exclusive_scan(local, carry, wsum);
        int bk = i0 / nchunks, ch = i0 - bk * nchunks;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            if (i0 + k < len) {
                cnt[i0 + k] = run;
                if (ch == 0) off_lds[bk] = run;   // first chunk of bucket bk
            }
            run += v[k];
            if (++ch == nchunks) {
                ch = 0;
                ++bk;
            }
        }
    }
    if (threadIdx.x == 0) off_lds[nbuckets] = carry;
    __syncthreads();
    write_tables(nbuckets, tile_m, off_lds, tiles_lds, wsum, offsets, tiles, tdesc);
    // scatter: chunk `wave` in pair order, 64 pairs per step (as bucket_scatter_kernel);
    // cnt[b][wave] is bucket b's next slot for this chunk
    if (!mine) return;   // no barrier follows
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int st = 0; st < kSmallSteps; ++st) {
        const int64_t p = base + st * 64 + lane;
        const bool live = p < pairs;
        const int32_t b = live ? bucket_of(idv[st], E) : -1;
        uint64_t same = __ballot(live);
#pragma unroll
        for (int k = 0; k < kKeyBits; ++k) {
            const uint64_t ones = __ballot(live && ((b >> k) & 1));
            same &= ((b >> k) & 1) ? ones : ~ones;
        }
        if (live) {
            const int rank = __popcll(same & below);
            int32_t* next = &cnt[b * nchunks + wave];
            const int32_t at = *next;
            sorted[at + rank] = (int32_t)p;
            wave_lds_fence();   // every lane has read its counter before the leaders update it
            if (rank == 0) *next = at + __popcll(same);
        }
        wave_lds_fence();
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
    // tile descriptors: at most sum over buckets of ceil(count / tile_m) tiles
    p.max_tiles = tile_m > 0 ? (pairs + p.buckets * (tile_m - 1)) / tile_m : 0;
    p.off_tdesc = off;   off = align(off + 16 * p.max_tiles);
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
    int4* tdesc = reinterpret_cast<int4*>(base + plan.off_tdesc);
    const int32_t nb = (int32_t)plan.buckets;
    if (plan.chunks <= kSmallChunks && (int64_t)nb * plan.chunks <= kSmallCounts && nb <= kSmallBuckets &&
        !route_split_forced()) {
        const size_t lds = sizeof(int32_t) * ((size_t)nb * plan.chunks + 2 * ((size_t)nb + 1));
        return launch("bucket_small_kernel", bucket_small_kernel, 1, kScanThreads, lds, s, ids, plan.pairs, (int32_t)E,
                      nb, (int32_t)plan.chunks, (int32_t)plan.tile_m, offsets, tiles, sorted, tdesc);
    }
    int st = launch("bucket_count_kernel", bucket_count_kernel, plan.chunks, kCountThreads,
                    sizeof(int32_t) * nb, s, ids, plan.pairs, (int32_t)E, nb, plan.chunks, counts);
    if (st != FTQ_OK) return st;
    st = launch("bucket_scan_kernel", bucket_scan_kernel, 1, kScanThreads, sizeof(int32_t) * 2 * (nb + 1), s,
                counts, plan.chunks, nb, (int32_t)plan.tile_m, offsets, tiles, tdesc);
    if (st != FTQ_OK) return st;
    return launch("bucket_scatter_kernel", bucket_scatter_kernel, (plan.chunks + kScatterWaves - 1) / kScatterWaves,
                  64 * kScatterWaves, sizeof(int32_t) * 2 * kScatterWaves * nb, s, ids, plan.pairs, (int32_t)E, nb,
                  plan.chunks, static_cast<const int32_t*>(counts), sorted);
}

}  // namespace ftq
