// Grouped path of the MoE expert matmul: expert-sorted tiles on int8 MFMA.
//
// After bucketing, the pairs routed to expert e occupy one contiguous segment
// of the sorted pair list.  Each workgroup computes one BM x BN output tile:
// BM pairs of one expert (a tile never straddles two experts; the last tile of
// an expert is ragged and its missing rows are masked, not padded in memory)
// against BN weight rows of that expert.  Prior art for this layout is the
// expert-sorted grouped GEMM of "Current Bug: CuTeDSLMoERunner" (Key
// Architecture: Fixed-Layout Padding; Bugs 2 and 4 for the tile -> expert
// lookup, done here as an upper-bound search over per-expert tile offsets);
// the tiles themselves are gfx950-native:
//   * K advances one 32-value quantisation block per v_mfma_i32_32x32x32_i8,
//     so each MFMA produces exactly the integer block partials P (exact int32);
//   * the Q4_0 nibbles are unpacked to signed bytes (q - 8) in registers while
//     the tile is staged to LDS; Q8_1 codes are gathered per pair row;
//   * per block the fp32 accumulator takes one FMA with the exact product of
//     the two fp16 scales: acc = fma(float(P), d4*d8, acc), blocks ascending.
//     The arithmetic per output element depends only on K, never on where the
//     pair sits in a tile, so results are batch invariant.
// The grid is a flat x axis over (M tile, N tile) with a grid-stride loop and
// 64-bit offsets; tiles past the device-side tile count exit at once.
#include "ftq_internal.h"

namespace ftq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBN = 128;        // weight rows per tile
constexpr int kKB = 4;          // quantisation blocks staged per pass
constexpr int kCodeStride = kKB * 32 + 16;   // LDS bytes per staged row of codes

struct GroupedParams {
    const uint8_t* w;
    const uint8_t* a;
    float* out;
    int32_t* partials;
    const int32_t* offsets;   // [E+2]
    const int32_t* tiles;     // [E+2]
    const int32_t* sorted;
    int64_t E, N, nb, top_k, nbuckets, n_tiles_n, work;   // work = max M tiles * N tiles
};

template <int BM>
struct Shape {
    static constexpr int WM = BM >= 64 ? 2 : 1;          // waves along M
    static constexpr int WN = 4 / WM;                    // waves along N
    static constexpr int SM = BM / (32 * WM);            // 32x32 sub-tiles per wave along M
    static constexpr int SN = kBN / (32 * WN);           // ... along N
    static_assert(SM >= 1 && SN >= 1, "tile shape");
};

__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Signed codes q - 8 for four nibbles held one per byte (values 0..15): set the
// top bit so the byte-wise subtract cannot borrow, then clear it again.
__device__ __forceinline__ uint32_t nibbles_minus_8(uint32_t x)
{
    return ((x | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
}

// Unpack one Q4_0 block given as fp16 scale bits and four words of nibbles.
__device__ __forceinline__ void store_block(uint8_t* codes, float* d4s, uint32_t dbits, const uint32_t qs[4])
{
    uint4 lo, hi;
    lo.x = nibbles_minus_8(qs[0] & 0x0f0f0f0fu);
    lo.y = nibbles_minus_8(qs[1] & 0x0f0f0f0fu);
    lo.z = nibbles_minus_8(qs[2] & 0x0f0f0f0fu);
    lo.w = nibbles_minus_8(qs[3] & 0x0f0f0f0fu);
    hi.x = nibbles_minus_8((qs[0] >> 4) & 0x0f0f0f0fu);
    hi.y = nibbles_minus_8((qs[1] >> 4) & 0x0f0f0f0fu);
    hi.z = nibbles_minus_8((qs[2] >> 4) & 0x0f0f0f0fu);
    hi.w = nibbles_minus_8((qs[3] >> 4) & 0x0f0f0f0fu);
    reinterpret_cast<uint4*>(codes)[0] = lo;
    reinterpret_cast<uint4*>(codes)[1] = hi;
    *d4s = half_bits_to_float(dbits);
}

template <int BM, int VEC, bool kPartials>
__global__ __launch_bounds__(kThreads) void moe_grouped_kernel(GroupedParams p)
{
    using S = Shape<BM>;
    __shared__ __align__(16) uint8_t a_codes[BM * kCodeStride];
    __shared__ __align__(16) uint8_t b_codes[kBN * kCodeStride];
    __shared__ __align__(16) float a_scale[kKB][BM];
    __shared__ __align__(16) float b_scale[kKB][kBN];
    __shared__ int32_t row_pair[BM];
    __shared__ int32_t row_tok[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int32_t total_tiles = p.tiles[p.nbuckets];

    for (int64_t work = blockIdx.x; work < p.work; work += gridDim.x) {
        const int64_t mt = work / p.n_tiles_n;
        const int64_t nt = work - mt * p.n_tiles_n;
        if (mt >= total_tiles) break;   // tiles are visited in increasing mt order

        // bucket of this M tile: the last b with tiles[b] <= mt
        int lo = 0, hi = (int)p.nbuckets;   // tiles[nbuckets] = total > mt
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.tiles[mid] <= mt) lo = mid; else hi = mid;
        }
        const int64_t bucket = lo;
        const int64_t slot0 = p.offsets[bucket] + (mt - p.tiles[bucket]) * BM;
        const int rows = (int)min<int64_t>(BM, p.offsets[bucket + 1] - slot0);
        const int64_t n0 = nt * kBN;

        __syncthreads();   // previous tile is done with the LDS row tables
        for (int m = tid; m < BM; m += kThreads) {
            const int32_t pid = m < rows ? p.sorted[slot0 + m] : 0;
            row_pair[m] = pid;
            row_tok[m] = (int32_t)(pid / p.top_k);
        }
        __syncthreads();

        if (bucket == p.E) {   // masked pairs: zero rows
            for (int i = tid; i < rows * kBN; i += kThreads) {
                const int m = i / kBN, n = i - m * kBN;
                if (n0 + n >= p.N) continue;
                const int64_t o = (int64_t)row_pair[m] * p.N + n0 + n;
                if constexpr (kPartials) {
                    for (int64_t b = 0; b < p.nb; ++b) p.partials[o * p.nb + b] = 0;
                } else {
                    p.out[o] = 0.0f;
                }
            }
            continue;
        }

        float acc[S::SM][S::SN][16];
#pragma unroll
        for (int i = 0; i < S::SM; ++i)
#pragma unroll
            for (int j = 0; j < S::SN; ++j)
#pragma unroll
                for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.0f;

        const uint8_t* wexp = p.w + (bucket * p.N) * p.nb * kQ4Bytes;

        for (int64_t kb0 = 0; kb0 < p.nb; kb0 += kKB) {
            __syncthreads();   // previous pass consumed
            // ---- stage A: BM pair rows x kKB blocks of Q8_1 -----------------
            for (int u = tid; u < BM * kKB; u += kThreads) {
                const int m = u / kKB, blk = u - m * kKB;
                const int64_t b = kb0 + blk;
                uint4 q0 = make_uint4(0, 0, 0, 0), q1 = q0;
                float d8 = 0.0f;
                if (m < rows && b < p.nb) {
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(p.a + ((int64_t)row_tok[m] * p.nb + b) * kQ8Bytes);
                    const uint32_t h = src[0];
                    q0 = make_uint4(src[1], src[2], src[3], src[4]);
                    q1 = make_uint4(src[5], src[6], src[7], src[8]);
                    d8 = half_bits_to_float(h & 0xffffu);
                }
                uint4* dst = reinterpret_cast<uint4*>(a_codes + m * kCodeStride + blk * 32);
                dst[0] = q0;
                dst[1] = q1;
                a_scale[blk][m] = d8;
            }
            // ---- stage B: kBN weight rows x kKB blocks of Q4_0 --------------
            if constexpr (VEC == 4) {
                // pairs of blocks: 36 bytes, 4-byte aligned (K/32 even, kb0 even)
                for (int u = tid; u < kBN * (kKB / 2); u += kThreads) {
                    const int n = u / (kKB / 2), bp = u - n * (kKB / 2);
                    const int64_t b = kb0 + 2 * bp;
                    uint32_t v[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
                    const bool ok_row = n0 + n < p.N;
                    if (ok_row && b < p.nb) {
                        const uint32_t* src = reinterpret_cast<const uint32_t*>(wexp + ((n0 + n) * p.nb + b) * kQ4Bytes);
#pragma unroll
                        for (int i = 0; i < 9; ++i) v[i] = src[i];
                    }
                    uint32_t qs[4];
                    qs[0] = __builtin_amdgcn_alignbit(v[1], v[0], 16);
                    qs[1] = __builtin_amdgcn_alignbit(v[2], v[1], 16);
                    qs[2] = __builtin_amdgcn_alignbit(v[3], v[2], 16);
                    qs[3] = __builtin_amdgcn_alignbit(v[4], v[3], 16);
                    if (!(ok_row && b < p.nb)) { qs[0] = qs[1] = qs[2] = qs[3] = 0x88888888u; }
                    store_block(b_codes + n * kCodeStride + (2 * bp) * 32, &b_scale[2 * bp][n], v[0] & 0xffffu, qs);
                    uint32_t qs1[4] = {v[5], v[6], v[7], v[8]};
                    if (!(ok_row && b + 1 < p.nb)) { qs1[0] = qs1[1] = qs1[2] = qs1[3] = 0x88888888u; v[4] = 0; }
                    store_block(b_codes + n * kCodeStride + (2 * bp + 1) * 32, &b_scale[2 * bp + 1][n], v[4] >> 16, qs1);
                }
            } else {
                // single blocks through 2-byte loads (odd K/32 or 2-byte aligned weights)
                for (int u = tid; u < kBN * kKB; u += kThreads) {
                    const int n = u / kKB, blk = u - n * kKB;
                    const int64_t b = kb0 + blk;
                    uint32_t dbits = 0, qs[4] = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                    if (n0 + n < p.N && b < p.nb) {
                        const uint16_t* src = reinterpret_cast<const uint16_t*>(wexp + ((n0 + n) * p.nb + b) * kQ4Bytes);
                        dbits = src[0];
#pragma unroll
                        for (int i = 0; i < 4; ++i) qs[i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
                    }
                    store_block(b_codes + n * kCodeStride + blk * 32, &b_scale[blk][n], dbits, qs);
                }
            }
            __syncthreads();

            // ---- MFMA + exact per-block rescale ----------------------------
            const int kblocks = (int)min<int64_t>(kKB, p.nb - kb0);
            for (int blk = 0; blk < kblocks; ++blk) {
                v4i af[S::SM], bf[S::SN];
#pragma unroll
                for (int i = 0; i < S::SM; ++i) {
                    const int m = (wm * S::SM + i) * 32 + (lane & 31);
                    af[i] = *reinterpret_cast<const v4i*>(a_codes + m * kCodeStride + blk * 32 + 16 * (lane >> 5));
                }
#pragma unroll
                for (int j = 0; j < S::SN; ++j) {
                    const int n = (wn * S::SN + j) * 32 + (lane & 31);
                    bf[j] = *reinterpret_cast<const v4i*>(b_codes + n * kCodeStride + blk * 32 + 16 * (lane >> 5));
                }
#pragma unroll
                for (int i = 0; i < S::SM; ++i) {
#pragma unroll
                    for (int j = 0; j < S::SN; ++j) {
                        v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                        const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], zero, 0, 0, 0);
                        const int nl = (wn * S::SN + j) * 32 + (lane & 31);
                        const float d4 = b_scale[blk][nl];
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int ml = (wm * S::SM + i) * 32 + 8 * g + 4 * (lane >> 5);
                            const float4 d8 = *reinterpret_cast<const float4*>(&a_scale[blk][ml]);
                            const float d8v[4] = {d8.x, d8.y, d8.z, d8.w};
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if constexpr (kPartials) {
                                    const int m = ml + r;
                                    const int64_t n = n0 + nl;
                                    if (m < rows && n < p.N)
                                        p.partials[((int64_t)row_pair[m] * p.N + n) * p.nb + kb0 + blk] = P[4 * g + r];
                                } else {
                                    acc[i][j][4 * g + r] = __builtin_fmaf((float)P[4 * g + r], d4 * d8v[r], acc[i][j][4 * g + r]);
                                }
                            }
                        }
                    }
                }
            }
        }

        if constexpr (!kPartials) {
#pragma unroll
            for (int i = 0; i < S::SM; ++i) {
#pragma unroll
                for (int j = 0; j < S::SN; ++j) {
                    const int64_t n = n0 + (wn * S::SN + j) * 32 + (lane & 31);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = (wm * S::SM + i) * 32 + 8 * g + 4 * (lane >> 5) + r;
                            if (m < rows && n < p.N) p.out[(int64_t)row_pair[m] * p.N + n] = acc[i][j][4 * g + r];
                        }
                    }
                }
            }
        }
    }
}

template <int BM, bool kPartials>
int launch_grouped(int vec, const GroupedParams& gp, int64_t grid, hipStream_t s)
{
    if (vec == 4)
        return launch("moe_grouped_kernel<4>", moe_grouped_kernel<BM, 4, kPartials>, grid, kThreads, 0, s, gp);
    return launch("moe_grouped_kernel<2>", moe_grouped_kernel<BM, 2, kPartials>, grid, kThreads, 0, s, gp);
}

}  // namespace

int64_t grouped_tile_m(const MoeArgs& m)
{
    // rows per M tile from the average pairs per expert (host arithmetic only)
    const int64_t per_expert = (m.T * m.top_k) / (m.E > 0 ? m.E : 1);
    if (per_expert >= 96) return 128;
    if (per_expert >= 40) return 64;
    return 32;
}

int run_grouped(const MoeArgs& m, const BucketPlan& plan, const void* ws, hipStream_t s)
{
    if (plan.pairs == 0) return FTQ_OK;
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    const uint8_t* base = static_cast<const uint8_t*>(ws);
    GroupedParams gp{};
    gp.w = static_cast<const uint8_t*>(m.w);
    gp.a = static_cast<const uint8_t*>(m.a);
    gp.out = m.out;
    gp.partials = m.partials;
    gp.offsets = reinterpret_cast<const int32_t*>(base + plan.off_offsets);
    gp.tiles = reinterpret_cast<const int32_t*>(base + plan.off_tiles);
    gp.sorted = reinterpret_cast<const int32_t*>(base + plan.off_sorted);
    gp.E = m.E;
    gp.N = m.N;
    gp.nb = m.K / kQK;
    gp.top_k = m.top_k;
    gp.nbuckets = plan.buckets;
    gp.n_tiles_n = (m.N + kBN - 1) / kBN;
    const int64_t bm = plan.tile_m;
    // sum over buckets of ceil(count/BM) <= (pairs + buckets*(BM-1)) / BM
    const int64_t max_mt = (plan.pairs + plan.buckets * (bm - 1)) / bm;
    gp.work = max_mt * gp.n_tiles_n;
    const int64_t grid = std::min<int64_t>(gp.work, lim.max_grid_x);
    const uintptr_t wa = reinterpret_cast<uintptr_t>(m.w);
    const int vec = (gp.nb % 2 == 0 && wa % 4 == 0) ? 4 : 2;
    const bool part = m.partials != nullptr;
    switch (bm) {
    case 128: return part ? launch_grouped<128, true>(vec, gp, grid, s) : launch_grouped<128, false>(vec, gp, grid, s);
    case 64: return part ? launch_grouped<64, true>(vec, gp, grid, s) : launch_grouped<64, false>(vec, gp, grid, s);
    default: return part ? launch_grouped<32, true>(vec, gp, grid, s) : launch_grouped<32, false>(vec, gp, grid, s);
    }
}

}  // namespace ftq
