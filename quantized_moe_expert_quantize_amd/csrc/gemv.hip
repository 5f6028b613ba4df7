// GEMV path of the MoE expert matmul: for few pairs per expert (decode).
//
// The same operation as the per-pair MoE GEMV of FreeToken PR #185 ("fix(kernel):
// launch GGUF MoE GEMV token axis on grid.x, not grid.z", Problem/Fix), laid out
// for gfx950 instead of one block per pair: a workgroup owns one expert and a
// tile of kRows weight rows, streams that tile from HBM exactly once, and serves
// every pair routed to the expert from it.  The weight stream is >97% of the
// bytes at decode sizes, so this is an HBM-bound kernel:
//   * the weight tile (kRows whole rows x kSeg blocks, contiguous in HBM) is
//     copied to LDS with the widest aligned vector loads the layout allows
//     (16 B when K/32 % 8 == 0), so HBM sees fully coalesced bursts even though
//     Q4_0 blocks are 18 bytes;
//   * the routed tokens' Q8_1 blocks are staged in LDS once per workgroup,
//     re-laid out as 16-byte aligned codes plus (d, -8*sum(q)) per block;
//   * 16 lanes share a row, each taking block pairs (36 bytes, 4-byte aligned in
//     LDS) in a fixed stride; per block the integer partial is 8 v_dot4_i32_i8
//     on the raw nibbles started from -8*sum(q8) (exact), then one fp32 FMA with
//     the exact scale product d4*d8; the 16 partial sums are combined with a
//     fixed xor-shuffle tree.  Nothing depends on the batch size, so a row's
//     bits do not change when the batch is split.
// The grid is one flat x axis over (expert bucket, row tile) with 64-bit
// index math; the pair list is either scanned from topk_ids by each
// workgroup (small batches) or read from the bucketed list.
#include "ftq_internal.h"

namespace ftq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 16;                         // weight rows per workgroup
constexpr int kLanesPerRow = kThreads / kRows;    // 16
constexpr int kSeg = 64;                          // K blocks staged per pass
constexpr int kPairChunk = 8;                     // pairs served per pass
constexpr int kRowStride = (kSeg * kQ4Bytes + 15) / 16 * 16 + 16;   // LDS bytes per staged row

struct GemvParams {
    const uint8_t* w;
    const uint8_t* a;
    const int32_t* ids;
    float* out;
    int32_t* partials;
    const int32_t* offsets;   // bucketed mode: [E+2] segment starts
    const int32_t* sorted;    // bucketed mode: pair ids grouped by bucket
    int64_t E, N, nb, top_k, pairs, row_tiles;
};

struct LdsLayout {
    int wt, aq, ad, plist, scan, bytes;
};

__host__ __device__ constexpr LdsLayout lds_layout(int scan_cap)
{
    LdsLayout l{};
    l.wt = 0;
    l.aq = l.wt + kRows * kRowStride;
    l.ad = l.aq + kPairChunk * kSeg * 32;
    l.plist = l.ad + kPairChunk * kSeg * 8;
    l.scan = l.plist + 2 * kPairChunk * 4 + 64;
    l.bytes = l.scan + scan_cap * 4;
    return l;
}

__device__ __forceinline__ int bucket_of(int32_t id, int64_t E) { return (id >= 0 && id < E) ? id : (int)E; }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Copy rows [n0, n0+rows) x blocks [sb, sb+len) of expert e into LDS.
template <int VEC>
__device__ __forceinline__ void stage_weights(const GemvParams& p, int64_t e, int64_t n0, int rows,
                                              int64_t sb, int len, uint8_t* wt)
{
    const int row_bytes = len * kQ4Bytes;
    const int upr = row_bytes / VEC;   // VEC divides row_bytes by construction
    for (int u = threadIdx.x; u < rows * upr; u += kThreads) {
        const int r = u / upr, col = u - r * upr;
        const uint8_t* src = p.w + ((e * p.N + n0 + r) * p.nb + sb) * kQ4Bytes + col * VEC;
        uint8_t* dst = wt + r * kRowStride + col * VEC;
        if constexpr (VEC == 16) {
            *reinterpret_cast<u32x4*>(dst) = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        } else if constexpr (VEC == 4) {
            *reinterpret_cast<uint32_t*>(dst) = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
        } else {
            *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
        }
    }
}

// Stage the Q8_1 blocks [sb, sb+len) of the chunk's tokens: codes as 32
// aligned bytes, and per block (d8 as float, -8 * sum of the codes).
__device__ __forceinline__ void stage_acts(const GemvParams& p, const int32_t* tok, int npc, int64_t sb,
                                           int len, uint8_t* aq, uint8_t* ad)
{
    for (int u = threadIdx.x; u < npc * len; u += kThreads) {
        const int j = u / len, blk = u - j * len;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(p.a + ((int64_t)tok[j] * p.nb + sb + blk) * kQ8Bytes);
        uint32_t v[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) v[i] = src[i];
        int sum = 0;
#pragma unroll
        for (int i = 1; i < 9; ++i) sum = __builtin_amdgcn_sdot4((int)v[i], 0x01010101, sum, false);
        uint4* q = reinterpret_cast<uint4*>(aq + (j * kSeg + blk) * 32);
        q[0] = make_uint4(v[1], v[2], v[3], v[4]);
        q[1] = make_uint4(v[5], v[6], v[7], v[8]);
        float2* dc = reinterpret_cast<float2*>(ad + (j * kSeg + blk) * 8);
        *dc = make_float2(half_bits_to_float(v[0] & 0xffffu), __int_as_float(-8 * sum));
    }
}

// Integer partial of one block: P = sum (nib - 8) * q8 = sum nib*q8 - 8*sum q8.
__device__ __forceinline__ int block_dot(const uint32_t qs[4], const uint4 a0, const uint4 a1, int neg8sum)
{
    int acc = neg8sum;
    acc = __builtin_amdgcn_sdot4((int)(qs[0] & 0x0f0f0f0fu), (int)a0.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)(qs[1] & 0x0f0f0f0fu), (int)a0.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)(qs[2] & 0x0f0f0f0fu), (int)a0.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)(qs[3] & 0x0f0f0f0fu), (int)a0.w, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((qs[0] >> 4) & 0x0f0f0f0fu), (int)a1.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((qs[1] >> 4) & 0x0f0f0f0fu), (int)a1.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((qs[2] >> 4) & 0x0f0f0f0fu), (int)a1.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((qs[3] >> 4) & 0x0f0f0f0fu), (int)a1.w, acc, false);
    return acc;
}

template <int VEC, bool kBucketed, bool kPartials>
__global__ __launch_bounds__(kThreads) void moe_gemv_kernel(GemvParams p, int scan_cap)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const LdsLayout L = lds_layout(scan_cap);
    uint8_t* wt = lds + L.wt;
    uint8_t* aq = lds + L.aq;
    uint8_t* ad = lds + L.ad;
    int32_t* plist = reinterpret_cast<int32_t*>(lds + L.plist);   // [kPairChunk] pair ids
    int32_t* ptok = plist + kPairChunk;                             // [kPairChunk] tokens
    int32_t* misc = ptok + kPairChunk;                              // counters
    int32_t* scan = reinterpret_cast<int32_t*>(lds + L.scan);

    const int64_t bid = blockIdx.x;
    const int64_t e = bid / p.row_tiles;               // bucket; e == E is the masked bucket
    const int64_t n0 = (bid - e * p.row_tiles) * kRows;
    const int rows = (int)min<int64_t>(kRows, p.N - n0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- the pair list of this bucket --------------------------------------
    const int32_t* list;
    int64_t count;
    if constexpr (kBucketed) {
        const int64_t beg = p.offsets[e];
        count = p.offsets[e + 1] - beg;
        list = p.sorted + beg;
    } else {
        if (tid == 0) misc[0] = 0;
        __syncthreads();
        for (int64_t base = 0; base < p.pairs; base += kThreads) {
            const int64_t q = base + tid;
            const bool match = q < p.pairs && bucket_of(p.ids[q], p.E) == e;
            const uint64_t m = __ballot(match);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (lane == 0) misc[2 + wave] = __popcll(m);
            __syncthreads();
            int off = misc[0];
            for (int w = 0; w < wave; ++w) off += misc[2 + w];
            if (match) scan[off + below] = (int32_t)q;
            __syncthreads();
            if (tid == 0) misc[0] += misc[2] + misc[3] + misc[4] + misc[5];
            __syncthreads();
        }
        count = misc[0];
        list = scan;
    }
    if (count == 0) return;

    const int r = tid / kLanesPerRow, l = tid % kLanesPerRow;
    const bool row_ok = r < rows;
    const int64_t n = n0 + r;

    for (int64_t c0 = 0; c0 < count; c0 += kPairChunk) {
        const int npc = (int)min<int64_t>(kPairChunk, count - c0);
        __syncthreads();   // the previous chunk is done with plist / LDS tiles
        if (tid < npc) {
            const int32_t pid = list[c0 + tid];
            plist[tid] = pid;
            ptok[tid] = (int32_t)(pid / p.top_k);
        }
        __syncthreads();

        if (e == p.E) {   // masked bucket: zero rows
            if (row_ok && l == 0) {
                for (int j = 0; j < npc; ++j) {
                    if constexpr (kPartials) {
                        for (int64_t b = 0; b < p.nb; ++b) p.partials[((int64_t)plist[j] * p.N + n) * p.nb + b] = 0;
                    } else {
                        p.out[(int64_t)plist[j] * p.N + n] = 0.0f;
                    }
                }
            }
            continue;
        }

        float acc[kPairChunk];
#pragma unroll
        for (int j = 0; j < kPairChunk; ++j) acc[j] = 0.0f;

        for (int64_t sb = 0; sb < p.nb; sb += kSeg) {
            const int len = (int)min<int64_t>(kSeg, p.nb - sb);
            if (sb > 0) __syncthreads();   // previous segment consumed
            stage_weights<VEC>(p, e, n0, rows, sb, len, wt);
            stage_acts(p, ptok, npc, sb, len, aq, ad);
            __syncthreads();
            if (row_ok) {
                const uint8_t* wrow = wt + r * kRowStride;
                for (int bp = l; 2 * bp < len; bp += kLanesPerRow) {
                    // two 18-byte blocks = nine 4-byte words, 4-byte aligned in LDS
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(wrow + 36 * bp);
                    uint32_t v[9];
#pragma unroll
                    for (int i = 0; i < 9; ++i) v[i] = src[i];
                    uint32_t qs[2][4];
                    float d4[2];
                    d4[0] = half_bits_to_float(v[0] & 0xffffu);
                    qs[0][0] = __builtin_amdgcn_alignbit(v[1], v[0], 16);
                    qs[0][1] = __builtin_amdgcn_alignbit(v[2], v[1], 16);
                    qs[0][2] = __builtin_amdgcn_alignbit(v[3], v[2], 16);
                    qs[0][3] = __builtin_amdgcn_alignbit(v[4], v[3], 16);
                    d4[1] = half_bits_to_float(v[4] >> 16);
                    qs[1][0] = v[5]; qs[1][1] = v[6]; qs[1][2] = v[7]; qs[1][3] = v[8];
                    const int nblk = min(2, len - 2 * bp);
                    for (int h = 0; h < nblk; ++h) {
                        const int blk = 2 * bp + h;
#pragma unroll
                        for (int j = 0; j < kPairChunk; ++j) {
                            if (j < npc) {
                                const uint4* aqb = reinterpret_cast<const uint4*>(aq + (j * kSeg + blk) * 32);
                                const float2 dc = *reinterpret_cast<const float2*>(ad + (j * kSeg + blk) * 8);
                                const int P = block_dot(qs[h], aqb[0], aqb[1], __float_as_int(dc.y));
                                if constexpr (kPartials) {
                                    p.partials[((int64_t)plist[j] * p.N + n) * p.nb + sb + blk] = P;
                                } else {
                                    acc[j] = __builtin_fmaf((float)P, d4[h] * dc.x, acc[j]);
                                }
                            }
                        }
                    }
                }
            }
        }
        if constexpr (!kPartials) {
#pragma unroll
            for (int j = 0; j < kPairChunk; ++j) {
                float v = acc[j];
                v += __shfl_xor(v, 8);
                v += __shfl_xor(v, 4);
                v += __shfl_xor(v, 2);
                v += __shfl_xor(v, 1);
                acc[j] = v;
            }
            if (row_ok && l == 0) {
                for (int j = 0; j < npc; ++j) p.out[(int64_t)plist[j] * p.N + n] = acc[j];
            }
        }
    }
}

template <bool kBucketed, bool kPartials>
int launch_gemv(int vec, const GemvParams& gp, int scan_cap, int64_t grid, size_t lds, hipStream_t s)
{
    switch (vec) {
    case 16: return launch("moe_gemv_kernel<16>", moe_gemv_kernel<16, kBucketed, kPartials>, grid, kThreads, lds, s, gp, scan_cap);
    case 4: return launch("moe_gemv_kernel<4>", moe_gemv_kernel<4, kBucketed, kPartials>, grid, kThreads, lds, s, gp, scan_cap);
    default: return launch("moe_gemv_kernel<2>", moe_gemv_kernel<2, kBucketed, kPartials>, grid, kThreads, lds, s, gp, scan_cap);
    }
}

}  // namespace

int run_gemv(const MoeArgs& m, const BucketPlan* plan, const void* ws, hipStream_t s)
{
    GemvParams gp{};
    gp.w = static_cast<const uint8_t*>(m.w);
    gp.a = static_cast<const uint8_t*>(m.a);
    gp.ids = m.ids;
    gp.out = m.out;
    gp.partials = m.partials;
    gp.E = m.E;
    gp.N = m.N;
    gp.nb = m.K / kQK;
    gp.top_k = m.top_k;
    gp.pairs = m.T * m.top_k;
    gp.row_tiles = (m.N + kRows - 1) / kRows;
    if (gp.pairs == 0) return FTQ_OK;
    const bool bucketed = plan != nullptr;
    int scan_cap = 0;
    if (bucketed) {
        const uint8_t* base = static_cast<const uint8_t*>(ws);
        gp.offsets = reinterpret_cast<const int32_t*>(base + plan->off_offsets);
        gp.sorted = reinterpret_cast<const int32_t*>(base + plan->off_sorted);
    } else {
        scan_cap = (int)gp.pairs;   // caller guarantees pairs <= kGemvScanMaxPairs
    }
    // widest copy unit that keeps every staged row segment aligned
    const uintptr_t wa = reinterpret_cast<uintptr_t>(m.w);
    int vec = 2;
    if (gp.nb % 8 == 0 && wa % 16 == 0) vec = 16;
    else if (gp.nb % 2 == 0 && wa % 4 == 0) vec = 4;
    const int64_t grid = (m.E + 1) * gp.row_tiles;
    const size_t lds = (size_t)lds_layout(scan_cap).bytes;
    if (bucketed) {
        return m.partials ? launch_gemv<true, true>(vec, gp, 0, grid, lds, s)
                          : launch_gemv<true, false>(vec, gp, 0, grid, lds, s);
    }
    return m.partials ? launch_gemv<false, true>(vec, gp, scan_cap, grid, lds, s)
                      : launch_gemv<false, false>(vec, gp, scan_cap, grid, lds, s);
}

}  // namespace ftq
