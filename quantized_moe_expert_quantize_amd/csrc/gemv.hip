// GEMV path of the MoE expert matmul: for few pairs per expert (decode).
//
// The same operation as the per-pair MoE GEMV of FreeToken PR #185 ("fix(kernel):
// launch GGUF MoE GEMV token axis on grid.x, not grid.z", Problem/Fix), laid out
// for gfx950 instead of one block per pair: each weight row of each routed
// expert is streamed from HBM exactly once and serves every pair routed to that
// expert.  At decode sizes the weight stream is >97% of the bytes, so this is an
// HBM-streaming kernel:
//   * work items are (routed expert, tile of 16 rows); the grid is what fits
//     on the device at once and each workgroup takes a contiguous share of the
//     items of equal cost, an item of an expert with c pairs costing 1-3 units
//     per pass over its weights plus c, so no workgroup waits for a second
//     round, every routed expert's rows are spread over all CUs, and experts
//     with more pairs get more CUs;
//   * 16 lanes share a row and walk it in steps of 16 groups of 8 Q4_0 blocks
//     (2304 bytes).  A step is loaded coalesced: each load instruction of the
//     16 lanes covers 256 contiguous bytes of the row (16 bytes per lane when
//     K/32 % 8 == 0), which the memory system serves at full rate, whereas
//     one 144-byte group per lane (lanes 144 bytes apart) reaches only about a
//     third of it.  The step then passes through a wave-private LDS buffer so
//     that lane l reads back its own group of 8 whole blocks; no workgroup
//     barrier is involved, and each wave issues the loads of its next step
//     before it computes the current one;
//   * the routed tokens' Q8_1 blocks are staged once per (expert, K segment) in
//     LDS as aligned codes plus (d, -8 * sum(q)), padded so that the 16 lanes
//     of a row (reading blocks 8 apart) hit distinct banks;
//   * per block the integer partial is 8 v_dot4_i32_i8 on the raw nibbles
//     started from -8*sum(q8) (exact), then one fp32 FMA with the exact scale
//     product d4*d8.  The summation order is fixed by the row alone: in each
//     step of 128 blocks a lane sums its 8 blocks in order from zero, the 16
//     lane sums are combined with a fixed xor-shuffle tree, and the step sums
//     are added in ascending order.  K segments (rows longer than the staging
//     budget, whose length depends on the batch) start and end on step
//     boundaries and continue the same running sum through the output, so a
//     row's bits depend neither on the grid nor on the batch: split halves of
//     a batch reproduce it bit for bit.
// The pair list of an expert is either scanned from topk_ids (small batches)
// or read from the bucketed list.  Masked pairs (ids outside [0, E)) form one
// more "expert" whose items write zero rows.
#include <type_traits>

#include "ftq_internal.h"

namespace ftq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLPR = 16;                                        // lanes per row
constexpr int kRowsPerWave = 64 / kLPR;                         // 4
constexpr int kRowsPerTile = kRowsPerWave * kWaves;             // 16
constexpr int kGroup = 8;                                       // blocks per lane group (8 blocks: 144 B for Q4_0)
constexpr int kPairChunk = 8;                                   // pairs served per pass
// Work split: a (bucket, row tile) item with c pairs costs `base` units per
// pass over its weights (one pass per chunk of at most pc_cap pairs) plus c,
// and each workgroup takes an equal share of the total cost, so that
// workgroups on experts with more pairs take fewer tiles.  Measured on decode
// shapes, streaming a tile's weights is worth about three pairs' dot products
// with two workgroups per CU and about one with three (more streams in flight).
constexpr int64_t kItemBase2PerCU = 3;
constexpr int64_t kItemBase3PerCU = 1;
__device__ __forceinline__ int64_t item_cost(int64_t c, int64_t pc_cap, int64_t base)
{
    // counts come from int32 offsets and pc_cap <= 8: 32-bit division suffices
    return base * (int64_t)(((uint32_t)c + (uint32_t)pc_cap - 1u) / (uint32_t)pc_cap) + c;
}
constexpr int kStepGroups = kLPR;                               // groups per row per step
constexpr int kStepBlocks = kStepGroups * kGroup;               // 128

// Weight block geometry per GGUF type (type ids as in GGUF files; Q4_0 = 2):
// bytes per block, per step of one row, per LDS row of a step (+16 B pad), per
// wave's rows.  A lane's group of 8 blocks is a multiple of 16 bytes for every
// type, so whole groups load as 16-byte units.
__host__ __device__ constexpr int w_block_bytes(int wt)
{
    return wt == FTQ_W_Q4_1 ? 20 : wt == FTQ_W_Q5_0 ? 22 : wt == FTQ_W_Q5_1 ? 24 : wt == FTQ_W_Q8_0 ? 34 : 18;
}
__host__ __device__ constexpr int step_bytes(int wt) { return kStepBlocks * w_block_bytes(wt); }
__host__ __device__ constexpr int wrow_pitch(int wt) { return step_bytes(wt) + 16; }
__host__ __device__ constexpr int wave_w(int wt) { return kRowsPerWave * wrow_pitch(wt); }
constexpr int kWavesPerSimd = 3;                                // register budget: 3 waves per SIMD
constexpr int64_t kLdsPerCU = 160 * 1024;
constexpr int64_t kTargetWGPerCU = 2;                           // LDS is sized so that 2 (or 3) workgroups fit

struct GemvParams {
    const uint8_t* w;
    const uint8_t* a;
    const int32_t* ids;
    float* out;
    int32_t* partials;
    const int32_t* offsets;   // bucketed mode: [E+2] segment starts
    const int32_t* sorted;    // bucketed mode: pair ids grouped by bucket
    int64_t E, N, nb, top_k, pairs, row_tiles;
    int64_t act_div;          // activation row of pair p: p / act_div
    int64_t half;             // fused activation: N/2 output columns (gate rows [0, half), up rows [half, N))
    int act;                  // fused activation: FTQ_ACT_*
    int64_t grid;             // workgroups launched
    int64_t seg;              // K blocks staged per pass (a multiple of 8)
    int pc_cap;               // activation rows staged per pass (<= kPairChunk)
    int64_t item_base;        // cost of one pass over a tile's weights, in pairs
    int list_cap;             // scan mode: LDS slots for the pair list
};

// Activation staging in LDS, block-major so that a lane's pairs sit at fixed
// offsets from one address: for block b of the segment and chunk row j (pc rows
// staged), 32 code bytes at code_off(b) + 32 j and an 8-byte entry (d8 as fp32,
// -8 * sum(q) as int32) at ent_off(b) + 8 j.  One 16-byte pad per 8 blocks
// (codes) and one 8-byte pad per 8 blocks (entries) put the blocks 8l+jb read
// by lanes l = 0..15 on distinct banks for any pc.
__host__ __device__ constexpr int64_t code_bytes(int64_t seg, int64_t pc) { return 32 * pc * seg + 16 * ((seg + 7) / 8) + 16; }
__host__ __device__ constexpr int64_t ent_bytes(int64_t seg, int64_t pc) { return 8 * pc * seg + 8 * ((seg + 7) / 8) + 8; }
__device__ __forceinline__ int code_off(int b, int pc) { return 32 * pc * b + 16 * (b >> 3); }
__device__ __forceinline__ int ent_off(int b, int pc) { return 8 * pc * b + 8 * (b >> 3); }

struct LdsLayout {
    int64_t wt, codes, ds, cnt, cost, wsum, plist, misc, list, bytes;
};

__host__ __device__ constexpr LdsLayout lds_layout(int wt, int64_t E, int64_t seg, int64_t pc_cap, int64_t list_cap)
{
    LdsLayout l{};
    l.wt = 0;
    l.codes = l.wt + kWaves * wave_w(wt);
    l.ds = l.codes + code_bytes(seg, pc_cap);
    l.cnt = (l.ds + ent_bytes(seg, pc_cap) + 15) / 16 * 16;   // [E+1] pairs per bucket
    l.cost = (l.cnt + 4 * (E + 1) + 7) / 8 * 8;              // [E+2] cost before each bucket
    l.wsum = l.cost + 8 * (E + 2);                            // [kWaves] scan partials
    l.plist = l.wsum + 8 * kWaves;
    l.misc = l.plist + 4 * 2 * kPairChunk;
    l.list = l.misc + 4 * 16;
    l.bytes = l.list + 4 * list_cap;
    return l;
}

__device__ __forceinline__ int64_t bucket_of(int32_t id, int64_t E) { return (id >= 0 && id < E) ? id : E; }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Stage the Q8_1 blocks [sb, sb+len) of the chunk's tokens.
__device__ __forceinline__ void stage_acts(const GemvParams& p, const int32_t* tok, int npc, int64_t sb, int len,
                                           uint8_t* codes, uint8_t* ds)
{
    for (int u = threadIdx.x; u < npc * len; u += kThreads) {
        const int j = u / len, b = u - j * len;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(p.a + ((int64_t)tok[j] * p.nb + sb + b) * kQ8Bytes);
        uint32_t v[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) v[i] = src[i];
        int sum = 0;
#pragma unroll
        for (int i = 1; i < 9; ++i) sum = __builtin_amdgcn_sdot4((int)v[i], 0x01010101, sum, false);
        u32x4* q = reinterpret_cast<u32x4*>(codes + code_off(b, p.pc_cap) + 32 * j);
        q[0] = u32x4{v[1], v[2], v[3], v[4]};
        q[1] = u32x4{v[5], v[6], v[7], v[8]};
        *reinterpret_cast<float2*>(ds + ent_off(b, p.pc_cap) + 8 * j) =
            make_float2(half_bits_to_float(v[0] & 0xffffu), __int_as_float(-8 * sum));
    }
}

// The 32-bit word at byte OFF (even) of a block pair held as words W.
template <int OFF>
__device__ __forceinline__ uint32_t word_at(const uint32_t* W)
{
    if constexpr (OFF % 4 == 0) return W[OFF / 4];
    else return __builtin_amdgcn_alignbit(W[OFF / 4 + 1], W[OFF / 4], 16);
}
template <int OFF>
__device__ __forceinline__ uint32_t half_at(const uint32_t* W)
{
    if constexpr (OFF % 4 == 0) return W[OFF / 4] & 0xffffu;
    else return W[OFF / 4] >> 16;
}

// Bits 0..3 of t moved to bit 4 of bytes 0..3 (the fifth bit of four codes):
// t * 0x204081 puts bit k at bit 8k with no carries.
__device__ __forceinline__ uint32_t high_bits(uint32_t t)
{
    return ((__builtin_amdgcn_ubfe(t, 0, 4) * 0x204081u) & 0x01010101u) << 4;
}

// One weight block at byte BASE of a pair's words, decoded once for all the
// pairs it serves: eight words of byte codes (c[i] pairs with activation
// codes 4i..4i+3, c[4+i] with 16+4i..), the fp16 bits of the scale and (offset
// types) of the offset.  Nibble byte i holds element i (low) and i + 16
// (high); qh bit i is bit 4 of element i; Q8_0 codes are the int8 bytes.
template <int WT, int BASE>
__device__ __forceinline__ void decode_block(const uint32_t* W, uint32_t c[8], uint32_t& dbits, uint32_t& mbits)
{
    dbits = half_at<BASE>(W);
    mbits = 0;
    if constexpr (WT == FTQ_W_Q8_0) {
        c[0] = word_at<BASE + 2>(W);  c[1] = word_at<BASE + 6>(W);
        c[2] = word_at<BASE + 10>(W); c[3] = word_at<BASE + 14>(W);
        c[4] = word_at<BASE + 18>(W); c[5] = word_at<BASE + 22>(W);
        c[6] = word_at<BASE + 26>(W); c[7] = word_at<BASE + 30>(W);
    } else {
        constexpr bool kOffset = WT == FTQ_W_Q4_1 || WT == FTQ_W_Q5_1;
        constexpr bool kFive = WT == FTQ_W_Q5_0 || WT == FTQ_W_Q5_1;
        constexpr int kQh = BASE + (kOffset ? 4 : 2);            // Q5 types: the 32 high bits
        constexpr int kQs = kQh + (kFive ? 4 : 0);               // the 16 nibble bytes
        if constexpr (kOffset) mbits = half_at<BASE + 2>(W);
        const uint32_t qs[4] = {word_at<kQs>(W), word_at<kQs + 4>(W), word_at<kQs + 8>(W), word_at<kQs + 12>(W)};
        uint32_t qh = 0;
        if constexpr (kFive) qh = word_at<kQh>(W);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = qs[i] & 0x0f0f0f0fu;
            c[4 + i] = (qs[i] >> 4) & 0x0f0f0f0fu;
            if constexpr (kFive) {
                c[i] |= high_bits(qh >> (4 * i));
                c[4 + i] |= high_bits(qh >> (16 + 4 * i));
            }
        }
    }
}

// The exact integer P = sum (q - z) q8 of a decoded block against one staged
// Q8_1 block (a0 = codes 0..15, a1 = 16..31; neg8sum = -8 * sum(q8)); the zero
// point z (8 for Q4_0, 16 for Q5_0, else 0) enters as the integer z * sum(q8).
template <int WT>
__device__ __forceinline__ int block_dot(const uint32_t c[8], const u32x4 a0, const u32x4 a1, int neg8sum)
{
    int acc = WT == FTQ_W_Q4_0 ? neg8sum : WT == FTQ_W_Q5_0 ? 2 * neg8sum : 0;
    acc = __builtin_amdgcn_sdot4((int)c[0], (int)a0.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[1], (int)a0.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[2], (int)a0.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[3], (int)a0.w, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[4], (int)a1.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[5], (int)a1.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[6], (int)a1.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)c[7], (int)a1.w, acc, false);
    return acc;
}

// One lane's share of a step as loaded: VEC-byte units 16*i + l of the step.
template <int VEC, int WT>
struct Raw {
    static constexpr int kUnits = step_bytes(WT) / VEC / kLPR;   // Q4_0: 9, 36 or 72
    static_assert(step_bytes(WT) % (VEC * kLPR) == 0, "whole units per lane");
    using Unit = typename std::conditional<VEC == 16, u32x4, typename std::conditional<VEC == 4, uint32_t, uint16_t>::type>::type;
    Unit u[kUnits];
};

// Load the step of `len` bytes at `src` (VEC-aligned, len a positive multiple
// of VEC).  Units past `len` re-read the last unit instead of branching, so the
// nine (or more) loads issue back to back with no wait between them.
template <int VEC, int WT>
__device__ __forceinline__ void load_step(const uint8_t* src, int len, int l, Raw<VEC, WT>& R)
{
    using Unit = typename Raw<VEC, WT>::Unit;
    const Unit* s = reinterpret_cast<const Unit*>(src);
    const int last = len / VEC - 1;
#pragma unroll
    for (int i = 0; i < Raw<VEC, WT>::kUnits; ++i) R.u[i] = __builtin_nontemporal_load(s + min(kLPR * i + l, last));
}

// Sum of v over the 16 lanes of a row, in every lane of the row.  Rotations of
// the row by 8, 4, 2 and 1 lanes (DPP, no LDS) pair each lane with the same
// partner values as the xor butterfly 8, 4, 2, 1 (after each level the values
// repeat with the next distance), so the bits equal that tree's.
__device__ __forceinline__ float row16_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));   // row_ror:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));   // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));   // row_ror:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));   // row_ror:1
    return v;
}

// Lanes of a wave exchange data through its private LDS step buffer.  The
// hardware keeps one wave's LDS accesses in order, but the compiler reasons per
// lane (a lane's own writes never overlap its own reads) and would move reads
// across the writes; a wave-scope fence orders them and costs no instruction
// beyond a wait for the LDS counter.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Write the loaded units to the row's LDS step buffer in memory order.  Units
// past the step's length land in the buffer's unused tail, which no lane reads
// as a block.
template <int VEC, int WT>
__device__ __forceinline__ void store_step(uint8_t* wrow, int l, const Raw<VEC, WT>& R)
{
    using Unit = typename Raw<VEC, WT>::Unit;
    Unit* d = reinterpret_cast<Unit*>(wrow);
#pragma unroll
    for (int i = 0; i < Raw<VEC, WT>::kUnits; ++i) d[kLPR * i + l] = R.u[i];
}

// Output column and weight row of lane row rw of wave `wave` in row tile t.
// Fused: a tile's 16 rows are the gate and up rows of 8 output columns; in
// wave w, row rw holds column 8t + 2w + (rw & 1), gate for rw < 2 and up for
// rw >= 2, so that after the row sums lane l holds the gate and lane l ^ 32
// the up value of the same column.
template <bool kFused>
__device__ __forceinline__ int64_t tile_col(int64_t t, int wave, int rw)
{
    if constexpr (kFused) return t * (kRowsPerTile / 2) + wave * (kRowsPerWave / 2) + (rw & 1);
    return t * kRowsPerTile + wave * kRowsPerWave + rw;
}
template <bool kFused>
__device__ __forceinline__ int64_t tile_row(const GemvParams& p, int64_t t, int wave, int rw)
{
    if constexpr (kFused) return (rw >> 1) * p.half + min<int64_t>(tile_col<kFused>(t, wave, rw), p.half - 1);
    return tile_col<kFused>(t, wave, rw);
}

// Rows of tiles [t0, t1) of expert e, K blocks [sb, sb+len), for the staged chunk.
// kMultiSeg: rows span several K segments, so later segments add to the sums
// already written (a global load inside the loop; kept out of the single
// segment case so that the weight loads are the only loads in flight there).
// NPC > 0: exactly NPC pairs are staged (no per-pair guards); NPC == 0: npc
// (1..8) pairs, guarded at run time.
// kFused: the rows of a tile are gate and up rows as tile_col describes.
// `stage` (the pair ids and the staged activation rows of the chunk, ending in
// a workgroup barrier) runs, for Q4_0, after the loads of the first weight
// step are issued, which do not depend on it, so that both are in flight
// together.
template <int VEC, bool kPartials, bool kMultiSeg, int NPC, bool kFused, int WT, typename Stage>
__device__ __forceinline__ void stream_tiles(const GemvParams& p, int64_t e, int64_t t0, int64_t t1, int64_t sb, int len,
                                             int npc, const int32_t* plist, uint8_t* wrow, const uint8_t* codes,
                                             const uint8_t* ds, int l, int rw, int wave, Stage&& stage)
{
    constexpr int kJ = NPC > 0 ? NPC : kPairChunk;
    const int pc = p.pc_cap;
    const int64_t nb = p.nb;
    constexpr int kBB = w_block_bytes(WT);
    constexpr int kPairWords = kBB / 2;   // two blocks, dword aligned in LDS
    const int64_t row_bytes = nb * kBB;
    const uint8_t* wexp = p.w + e * p.N * row_bytes;
    const int64_t gbeg = sb / kGroup, gend = (sb + len + kGroup - 1) / kGroup;
    const int64_t seg_end = (sb + len) * kBB;   // row bytes up to the segment's end
    auto step_len = [&](int64_t ws) { return (int)min<int64_t>(step_bytes(WT), seg_end - ws * kGroup * kBB); };
    // output column of this lane's row in tile t (the weight row unless fused)
    auto col_of = [&](int64_t t) { return tile_col<kFused>(t, wave, rw); };
    auto row_of = [&](int64_t t) { return tile_row<kFused>(p, t, wave, rw); };
    // rows past N (last tile only) load row N-1; their sums are never written
    auto src_of = [&](int64_t t, int64_t ws) {
        return wexp + min<int64_t>(row_of(t), p.N - 1) * row_bytes + ws * kGroup * kBB;
    };

    // steps are (tile t, first group ws of the step), tile-major
    auto advance = [&](int64_t& t, int64_t& ws) {
        ws += kStepGroups;
        if (ws >= gend) {
            ws = gbeg;
            ++t;
        }
    };

    float acc[kJ];   // this lane's sum over its blocks of the current step
    float rs[kJ];    // the row's running sum over the steps so far
#pragma unroll
    for (int j = 0; j < kJ; ++j) acc[j] = rs[j] = 0.0f;

    // Steps: (tile t, first group ws of the step); the loads of the next step
    // are in flight while the current one is computed.  The last step of the
    // range loads nothing more (a wave-uniform branch): the weight loads are
    // non-temporal, so a re-read of an earlier step would go to HBM again.
    Raw<VEC, WT> R;
    int64_t t = t0, ws = gbeg;
    auto load = [&](int64_t tl, int64_t wl) __attribute__((always_inline)) {
        load_step<VEC>(src_of(tl, wl), step_len(wl), l, R);
    };
    if constexpr (WT == FTQ_W_Q4_0) {
        load(t, ws);
        stage();
    } else {
        // the wider blocks' step buffers would stay live through the staging
        // and spill: stage first
        stage();
        load(t, ws);
    }
    while (t < t1) {
        const int64_t n = kFused ? col_of(t) : row_of(t);
        if constexpr (kMultiSeg && !kPartials) {
            // a later K segment continues the running sum that the earlier
            // segments left in the output (same order as one segment)
            if (sb > 0 && ws == gbeg) {
#pragma unroll
                for (int j = 0; j < kJ; ++j)
                    rs[j] = (n < p.N && (NPC > 0 || j < npc)) ? p.out[(int64_t)plist[j] * p.N + n] : 0.0f;
            }
        }
        wave_lds_fence();   // the previous step's reads of the buffer come first
        store_step<VEC>(wrow, l, R);
        wave_lds_fence();   // and this step's writes before its reads
        int64_t t2 = t, ws2 = ws;
        advance(t2, ws2);
        if (t2 < t1) load(t2, ws2);
        // lanes whose group is past the segment (partial steps) compute on a
        // valid group with scale 0 (fma(P, 0, acc) == acc); rows past N are
        // never written
        const int64_t g = ws + l;
        const bool valid = g < gend;
        const int64_t gl = (valid ? g : gend - 1) - gbeg;   // group within the segment
        {
            // 16-byte loads imply K/32 % 8 == 0: every group is whole
            const int nblk = VEC == 16 ? kGroup : (int)min<int64_t>(kGroup, nb - (gbeg + gl) * kGroup);
            const int bl0 = (int)(gl * kGroup);   // first block of the group in the segment
            const uint32_t* gw = reinterpret_cast<const uint32_t*>(wrow + l * kGroup * kBB);
            // block pairs are read from the step buffer one at a time, which
            // bounds what is live at once to two blocks
#pragma unroll
            for (int jp = 0; jp < kGroup / 2; ++jp) {
                uint32_t bp[kPairWords];
#pragma unroll
                for (int i = 0; i < kPairWords; ++i) bp[i] = gw[kPairWords * jp + i];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int jb = 2 * jp + h;
                    if (VEC == 16 || jb < nblk) {
                        uint32_t cw[8], dbits, mbits;
                        if (h == 0) decode_block<WT, 0>(bp, cw, dbits, mbits);
                        else decode_block<WT, kBB>(bp, cw, dbits, mbits);
                        // lanes past the segment add P * 0 (and S * 0)
                        const float d4 = valid ? half_bits_to_float(dbits) : 0.0f;
                        const float m4 = valid ? half_bits_to_float(mbits) : 0.0f;
                        const uint8_t* cbj = codes + code_off(bl0 + jb, pc);
                        const uint8_t* ebj = ds + ent_off(bl0 + jb, pc);
#pragma unroll
                        for (int j = 0; j < kJ; ++j) {
                            if (NPC > 0 || j < npc) {
                                const u32x4* aqb = reinterpret_cast<const u32x4*>(cbj + 32 * j);
                                const float2 en = *reinterpret_cast<const float2*>(ebj + 8 * j);
                                const int neg8sum = __float_as_int(en.y);
                                const int P = block_dot<WT>(cw, aqb[0], aqb[1], neg8sum);
                                if constexpr (kPartials) {
                                    if (valid && n < p.N)
                                        p.partials[((int64_t)plist[j] * p.N + n) * nb + sb + bl0 + jb] = P;
                                } else {
                                    acc[j] = __builtin_fmaf((float)P, d4 * en.x, acc[j]);
                                    if constexpr (WT == FTQ_W_Q4_1 || WT == FTQ_W_Q5_1)   // + m d8 sum(q8)
                                        acc[j] = __builtin_fmaf((float)(-(neg8sum >> 3)), m4 * en.x, acc[j]);
                                }
                            }
                        }
                    }
                }
            }
        }
        if constexpr (!kPartials) {
            // end of a step: the 16 lane sums by a fixed tree (row16_sum: every
            // lane of the row gets the same value), added to the row's running sum
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                const float v = row16_sum(acc[j]);
                acc[j] = 0.0f;
                const bool first = ws == gbeg && !(kMultiSeg && sb > 0);
                rs[j] = first ? v : rs[j] + v;
            }
        }
        if (t2 != t) {   // the tile's rows are complete (wave-uniform)
            if constexpr (kFused) {
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    const float v = rs[j];
                    const float up = __shfl_xor(v, 32);
                    if (n < p.half && rw < 2 && l == 0 && (NPC > 0 || j < npc))
                        p.out[(int64_t)plist[j] * p.half + n] = gated_act(p.act, v) * up;
                }
            } else if constexpr (!kPartials) {
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    if (n < p.N && l == 0 && (NPC > 0 || j < npc)) p.out[(int64_t)plist[j] * p.N + n] = rs[j];
                }
            }
        }
        t = t2;
        ws = ws2;
    }
}

template <int VEC, bool kBucketed, bool kPartials, bool kMultiSeg, bool kFused, int WT>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void moe_gemv_kernel(GemvParams p)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int64_t nb = p.nb;
    const LdsLayout L = lds_layout(WT, p.E, p.seg, p.pc_cap, p.list_cap);
    uint8_t* codes = lds + L.codes;
    uint8_t* ds = lds + L.ds;
    int32_t* cnt = reinterpret_cast<int32_t*>(lds + L.cnt);         // pairs per bucket (E+1)
    int64_t* cost = reinterpret_cast<int64_t*>(lds + L.cost);       // cost of the buckets before b (E+2)
    int64_t* wsum = reinterpret_cast<int64_t*>(lds + L.wsum);       // per-wave scan totals
    int32_t* plist = reinterpret_cast<int32_t*>(lds + L.plist);     // [kPairChunk] pair ids
    int32_t* ptok = plist + kPairChunk;                               // [kPairChunk] tokens
    int32_t* misc = reinterpret_cast<int32_t*>(lds + L.misc);
    int32_t* slist = reinterpret_cast<int32_t*>(lds + L.list);      // scan mode: the expert's pairs

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l = lane % kLPR, rw = lane / kLPR;   // lane within the row, row within the wave
    // scan mode: the first kThreads ids are read once, into registers, and
    // serve both the bucket counts and the pair lists
    int32_t id0 = -1;
    if constexpr (!kBucketed) {
        if (tid < p.pairs) id0 = p.ids[tid];
    }

    // ---- pairs per bucket (experts, and E for masked pairs) ------------------
    if constexpr (kBucketed) {
        for (int64_t b = tid; b <= p.E; b += kThreads) cnt[b] = p.offsets[b + 1] - p.offsets[b];
    } else {
        for (int64_t b = tid; b <= p.E; b += kThreads) cnt[b] = 0;
        __syncthreads();
        for (int64_t q = tid; q < p.pairs; q += kThreads) {
            const int32_t id = q < kThreads ? id0 : p.ids[q];
            atomicAdd(&cnt[bucket_of(id, p.E)], 1);
        }
    }
    __syncthreads();

    // ---- exclusive prefix of the bucket costs (row_tiles * item_cost) ----------
    auto wave_incl_scan = [&](int64_t v) __attribute__((always_inline)) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t u = __shfl_up(v, o);
            if (lane >= o) v += u;
        }
        return v;
    };
    if (p.E < 64) {   // one wave holds every bucket
        if (wave == 0) {
            const int32_t c = lane <= p.E ? cnt[lane] : 0;
            const int64_t v = c > 0 ? p.row_tiles * item_cost(c, p.pc_cap, p.item_base) : 0;
            const int64_t incl = wave_incl_scan(v);
            if (lane <= p.E) cost[lane] = incl - v;
            if (lane == p.E) cost[p.E + 1] = incl;
        }
        __syncthreads();
    }
    int64_t carry = 0;
    for (int64_t base = 0; p.E >= 64 && base <= p.E; base += kThreads) {
        const int64_t b = base + tid;
        const int32_t c = b <= p.E ? cnt[b] : 0;
        const int64_t v = c > 0 ? p.row_tiles * item_cost(c, p.pc_cap, p.item_base) : 0;
        const int64_t incl = wave_incl_scan(v);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int64_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? wsum[w] : 0;
            total += wsum[w];
        }
        if (b <= p.E) cost[b] = carry + before + incl - v;
        if (b == p.E) cost[p.E + 1] = carry + before + incl;
        carry += total;
        __syncthreads();   // wsum is rewritten by the next chunk; cost is read after the loop
    }

    // ---- this workgroup's share of the cost: the items starting in [x0, x1) ---
    // Boundaries only need to be the same monotone function of the workgroup
    // index on both sides of each boundary (0 at the first, C at the last), so
    // they are computed in double (exact for these magnitudes) and the item
    // bounds with 32-bit division when the total fits: 64-bit integer
    // division is a long software sequence on the GPU.
    const int64_t C = uniform(cost[p.E + 1]);
    auto share = [&](int64_t g) { return (int64_t)((double)g * (double)C / (double)p.grid); };
    const int64_t x0 = share(blockIdx.x), x1 = share((int64_t)blockIdx.x + 1);
    if (x0 >= x1) return;
    const bool narrow = C < (int64_t(1) << 31);
    auto ceil_div = [&](int64_t a, int64_t b) -> int64_t {   // a >= 0, 0 < b <= C
        if (narrow) return (int64_t)(((uint32_t)a + (uint32_t)b - 1u) / (uint32_t)b);
        return (a + b - 1) / b;
    };
    int64_t e_first = 0;
    {
        int64_t lo = 0, hi = p.E;   // the last bucket whose cost starts at or before x0
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            if (cost[mid] <= x0) lo = mid; else hi = mid - 1;
        }
        e_first = uniform((int32_t)lo);
    }

    for (int64_t e = e_first; e <= p.E && cost[e] < x1; ++e) {
        const int64_t c = cnt[e];
        if (c == 0) continue;
        const int64_t ci = item_cost(c, p.pc_cap, p.item_base), ce = cost[e];
        // item t of bucket e starts at ce + t * ci
        const int64_t t0 = uniform((int32_t)(x0 > ce ? ceil_div(x0 - ce, ci) : 0));
        const int64_t t1 = uniform((int32_t)min<int64_t>(p.row_tiles, ceil_div(x1 - ce, ci)));
        if (t0 >= t1) continue;

        // ---- the pair list of this bucket ----------------------------------
        const int32_t* list;
        int64_t count;
        __syncthreads();   // the previous bucket is done with the list and the staged rows
        if constexpr (kBucketed) {
            const int64_t beg = uniform(p.offsets[e]);
            count = uniform(p.offsets[e + 1]) - beg;
            list = p.sorted + beg;
        } else {
            if (tid == 0) misc[0] = 0;
            __syncthreads();
            for (int64_t base = 0; base < p.pairs; base += kThreads) {
                const int64_t q = base + tid;
                const bool match = q < p.pairs && bucket_of(base == 0 ? id0 : p.ids[q], p.E) == e;
                const uint64_t mb = __ballot(match);
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0));
                if (lane == 0) misc[2 + wave] = __popcll(mb);
                __syncthreads();
                int off = misc[0];
                for (int w = 0; w < wave; ++w) off += misc[2 + w];
                if (match) slist[off + below] = (int32_t)q;
                __syncthreads();
                if (tid == 0) misc[0] += misc[2] + misc[3] + misc[4] + misc[5];
                __syncthreads();
            }
            count = uniform(misc[0]);
            list = slist;
        }

        for (int64_t c0 = 0; c0 < count; c0 += p.pc_cap) {
            const int npc = (int)min<int64_t>(p.pc_cap, count - c0);
            // the chunk's pair ids and tokens (after the previous chunk is done
            // with them and with the staged rows)
            auto chunk_ids = [&]() __attribute__((always_inline)) {
                __syncthreads();
                if (tid < npc) {
                    const int32_t pid = list[c0 + tid];
                    plist[tid] = pid;
                    ptok[tid] = (int32_t)(pid / p.act_div);
                }
                __syncthreads();
            };

            if (e == p.E) {   // masked bucket: zero outputs of tiles [t0, t1)
                chunk_ids();
                constexpr int64_t kCols = kFused ? kRowsPerTile / 2 : kRowsPerTile;
                const int64_t width = kFused ? p.half : p.N;
                const int64_t r0 = t0 * kCols, r1 = min<int64_t>(t1 * kCols, width);
                for (int64_t i = tid; i < (int64_t)npc * (r1 - r0); i += kThreads) {
                    const int j = (int)(i / (r1 - r0));
                    const int64_t n = r0 + (i - (int64_t)j * (r1 - r0));
                    if constexpr (kPartials) {
                        for (int64_t b = 0; b < nb; ++b) p.partials[((int64_t)plist[j] * p.N + n) * nb + b] = 0;
                    } else {
                        p.out[(int64_t)plist[j] * width + n] = 0.0f;
                    }
                }
                continue;
            }

            // K segments: one unless the staged rows would not fit the budget.
            for (int64_t sb = 0; sb < nb; sb += p.seg) {
                const int len = (int)min<int64_t>(p.seg, nb - sb);
                // run by stream_tiles once its first weight loads are out
                auto stage = [&]() __attribute__((always_inline)) {
                    if (sb == 0) chunk_ids();
                    else __syncthreads();   // the previous segment's activations are consumed
                    stage_acts(p, ptok, npc, sb, len, codes, ds);
                    __syncthreads();
                };
                uint8_t* wrow = lds + L.wt + wave * wave_w(WT) + rw * wrow_pitch(WT);
#define FTQ_STREAM(NPC) stream_tiles<VEC, kPartials, kMultiSeg, NPC, kFused, WT>(p, e, t0, t1, sb, len, npc, plist, wrow, codes, ds, l, rw, wave, stage)
                // a stream without per-pair guards for each pair count up to 4
                // (and up to 8 in the plain Q4_0 kernel that scans the ids, the
                // one the path rule gives such counts: the other kernels would
                // spill with them); other counts keep the guarded loop, whose
                // guards also stop the scheduler from interleaving all 8 blocks
                // (which would need 8 * 10 * npc registers)
                constexpr bool kWideNpc = VEC == 16 && WT == FTQ_W_Q4_0 && !kFused && !kPartials && !kBucketed;
                if (VEC == 16 && npc == 1) {
                    FTQ_STREAM(1);
                } else if (VEC == 16 && npc == 2) {
                    FTQ_STREAM(2);
                } else if (VEC == 16 && npc == 3) {
                    FTQ_STREAM(3);
                } else if (VEC == 16 && npc == 4) {
                    FTQ_STREAM(4);
                } else if (kWideNpc && npc == 5) {
                    FTQ_STREAM(5);
                } else if (kWideNpc && npc == 6) {
                    FTQ_STREAM(6);
                } else if (kWideNpc && npc == 7) {
                    FTQ_STREAM(7);
                } else if (kWideNpc && npc == 8) {
                    FTQ_STREAM(8);
                } else {
                    FTQ_STREAM(0);
                }
#undef FTQ_STREAM
            }
        }
    }
}

template <int VEC, bool kBucketed, bool kPartials, int WT>
int launch_seg(bool multi, const GemvParams& gp, size_t lds, hipStream_t s)
{
    if constexpr (!kPartials && WT == FTQ_W_Q4_0) {   // a fused activation needs whole rows (one K segment)
        if (gp.act != 0)
            return launch("moe_gemv_kernel<act>", moe_gemv_kernel<VEC, kBucketed, false, false, true, WT>, gp.grid,
                          kThreads, lds, s, gp);
    }
    if (multi)
        return launch("moe_gemv_kernel", moe_gemv_kernel<VEC, kBucketed, kPartials, true, false, WT>, gp.grid, kThreads,
                      lds, s, gp);
    return launch("moe_gemv_kernel", moe_gemv_kernel<VEC, kBucketed, kPartials, false, false, WT>, gp.grid, kThreads,
                  lds, s, gp);
}

template <bool kBucketed, bool kPartials, int WT>
int launch_gemv(int vec, const GemvParams& gp, size_t lds, hipStream_t s)
{
    const bool multi = gp.seg < gp.nb;
    switch (vec) {
    case 16: return launch_seg<16, kBucketed, kPartials, WT>(multi, gp, lds, s);
    case 4: return launch_seg<4, kBucketed, kPartials, WT>(multi, gp, lds, s);
    default:
        if constexpr (WT == FTQ_W_Q4_0) return launch_seg<2, kBucketed, kPartials, WT>(multi, gp, lds, s);
        set_error("internal: 2-byte weight loads are built for Q4_0 only");
        return FTQ_ERR_UNSUPPORTED;
    }
}

template <bool kBucketed, bool kPartials>
int launch_wtype(int wtype, int vec, const GemvParams& gp, size_t lds, hipStream_t s)
{
    switch (wtype) {
    case FTQ_W_Q4_1: return launch_gemv<kBucketed, kPartials, FTQ_W_Q4_1>(vec, gp, lds, s);
    case FTQ_W_Q5_0: return launch_gemv<kBucketed, kPartials, FTQ_W_Q5_0>(vec, gp, lds, s);
    case FTQ_W_Q5_1: return launch_gemv<kBucketed, kPartials, FTQ_W_Q5_1>(vec, gp, lds, s);
    case FTQ_W_Q8_0: return launch_gemv<kBucketed, kPartials, FTQ_W_Q8_0>(vec, gp, lds, s);
    default: return launch_gemv<kBucketed, kPartials, FTQ_W_Q4_0>(vec, gp, lds, s);
    }
}

}  // namespace

GemvPlan plan_gemv(const MoeArgs& m, bool bucketed)
{
    GemvPlan g{};
    const int64_t nb = m.K / kQK;
    const int64_t pairs = m.T * m.top_k;
    g.list_cap = bucketed ? 0 : pairs;   // scan mode: the caller keeps pairs <= kGemvScanMaxPairs
    // a bucket never holds more than T*top_k pairs
    g.pc_cap = std::min<int64_t>(kPairChunk, std::max<int64_t>(pairs, 1));
    // K segment: whole rows when the staged activations fit next to the weight
    // buffers with the chosen workgroups per CU (below), else the largest
    // multiple of a step (128 blocks) that fits, so that every step is full
    const int64_t fixed = lds_layout(m.wtype, m.E, 0, 0, g.list_cap).bytes;
    auto act_bytes_pc = [&](int64_t seg, int64_t pc) { return code_bytes(seg, pc) + ent_bytes(seg, pc); };
    auto act_bytes = [&](int64_t seg) { return act_bytes_pc(seg, g.pc_cap); };
    const int64_t avg_pairs = std::max<int64_t>(1, (pairs + m.E - 1) / m.E);
    // Three workgroups per CU (more streams in flight) when whole activation
    // rows of the pairs an expert is likely to hold still fit, at least
    // max(4, 2 * the average per expert) of them, so that an expert's weights
    // are still streamed once; else two, with more pairs per pass.
    int64_t budget = std::max<int64_t>(kLdsPerCU / kTargetWGPerCU - fixed, 0);
    {
        const int64_t budget3 = std::max<int64_t>(kLdsPerCU / 3 - fixed, 0);
        int64_t pc3 = g.pc_cap;
        while (pc3 > 1 && act_bytes_pc(nb, pc3) > budget3) --pc3;
        const int64_t want = std::min<int64_t>(g.pc_cap, std::max<int64_t>(4, 2 * avg_pairs));
        if (act_bytes_pc(nb, pc3) <= budget3 && pc3 >= want) budget = budget3;
    }
    // fewer pairs per pass, down to the average per expert, rather than one
    // workgroup per CU (larger weight blocks leave less room for the rows)
    while (g.pc_cap > avg_pairs && act_bytes(nb) > budget) --g.pc_cap;
    if (m.act) {
        // the activation is applied once a row's sum is complete: stage whole
        // rows, with fewer pairs per pass if need be
        while (g.pc_cap > 1 && act_bytes(nb) > budget) --g.pc_cap;
        if (act_bytes(nb) > budget) {
            g.fits = false;
            return g;
        }
    }
    if (act_bytes(nb) <= budget) {
        g.seg = nb;
    } else {
        int64_t seg = kStepBlocks;
        while (seg + kStepBlocks < nb && act_bytes(seg + kStepBlocks) <= budget) seg += kStepBlocks;
        g.seg = seg;
    }
    g.lds = lds_layout(m.wtype, m.E, g.seg, g.pc_cap, g.list_cap).bytes;
    // workgroups resident per CU (LDS and registers permitting)
    const int64_t by_lds = std::max<int64_t>(1, kLdsPerCU / g.lds);
    g.per_cu = std::min<int64_t>(by_lds, kWavesPerSimd * 4 / kWaves);
    g.item_base = g.per_cu >= 3 ? kItemBase3PerCU : kItemBase2PerCU;
    g.fits = true;
    return g;
}

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
    gp.act_div = m.act_div;
    gp.pairs = m.T * m.top_k;
    gp.act = m.act;
    gp.half = m.act ? m.N / 2 : 0;
    // fused: 8 output columns (their 8 gate and 8 up rows) per tile
    gp.row_tiles = m.act ? (gp.half + kRowsPerTile / 2 - 1) / (kRowsPerTile / 2) : (m.N + kRowsPerTile - 1) / kRowsPerTile;
    if (gp.pairs == 0) return FTQ_OK;
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    const bool bucketed = plan != nullptr;
    if (bucketed) {
        const uint8_t* base = static_cast<const uint8_t*>(ws);
        gp.offsets = reinterpret_cast<const int32_t*>(base + plan->off_offsets);
        gp.sorted = reinterpret_cast<const int32_t*>(base + plan->off_sorted);
    }
    const GemvPlan g = plan_gemv(m, bucketed);
    if (!g.fits) {
        set_error("fused activation on the GEMV path: one activation row of K = %lld does not fit on chip",
                  (long long)m.K);
        return FTQ_ERR_UNSUPPORTED;
    }
    gp.list_cap = (int)g.list_cap;
    gp.pc_cap = (int)g.pc_cap;
    gp.seg = g.seg;
    gp.item_base = g.item_base;
    const int64_t lds = g.lds;
    const int64_t max_items = (std::min<int64_t>(m.E, gp.pairs) + 1) * gp.row_tiles;
    gp.grid = std::max<int64_t>(1, std::min<int64_t>((int64_t)lim.cu_count * g.per_cu, max_items));
    // widest load unit that keeps every step aligned: 16 bytes when K/32 is a
    // multiple of 8 (whole lane groups), 4 when every block boundary that a
    // step starts or ends on is 4-byte aligned, else 2 (Q4_0 only)
    const int64_t bb = w_block_bytes(m.wtype);
    const uintptr_t wa = reinterpret_cast<uintptr_t>(m.w);
    int vec = 2;
    if (gp.nb % 8 == 0 && wa % 16 == 0) vec = 16;
    else if ((bb % 4 == 0 || gp.nb % 2 == 0) && wa % 4 == 0) vec = 4;
    if (vec == 2 && m.wtype != FTQ_W_Q4_0) {
        set_error("weight type %d needs 4-byte aligned weight rows (K/32 even, or 4-byte blocks)", m.wtype);
        return FTQ_ERR_UNSUPPORTED;
    }
    if (bucketed) {
        return m.partials ? launch_wtype<true, true>(m.wtype, vec, gp, (size_t)lds, s)
                          : launch_wtype<true, false>(m.wtype, vec, gp, (size_t)lds, s);
    }
    return m.partials ? launch_wtype<false, true>(m.wtype, vec, gp, (size_t)lds, s)
                      : launch_wtype<false, false>(m.wtype, vec, gp, (size_t)lds, s);
}

}  // namespace ftq
