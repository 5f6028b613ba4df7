// Grouped path of the MoE expert matmul: expert-sorted tiles on the matrix cores.
//
// After bucketing, the pairs routed to expert e occupy one contiguous segment
// of the sorted pair list.  Each workgroup computes one BM x 128 output tile:
// BM pairs of one expert (a tile never straddles two experts; the last tile of
// an expert is ragged and its missing rows are masked, not padded in memory)
// against 128 weight rows of that expert.  Prior art for this layout is the
// expert-sorted grouped GEMM of "Current Bug: CuTeDSLMoERunner" (Key
// Architecture: Fixed-Layout Padding; Bugs 2 and 4 for the tile -> expert
// lookup, done here as an upper-bound search over per-expert tile offsets).
//
// Arithmetic, exact at every step.  Per output element and quantisation block b
// the result needs the integer partial P_b = sum_i (q4-8)*q8 and the scale
// product d4*d8; the vector ALUs then do a single fp32 FMA per element and
// block, acc = fma(P_b, d4*d8, acc), blocks in ascending order.  P_b comes from
// the matrix cores in one of two formulations, which give the same bits:
//   * int8 (the default): one v_mfma_i32_32x32x32_i8 per 32x32 sub-tile and
//     block on the int8 codes (weight nibbles unpacked to q - 8 while staging,
//     Q8_1 codes staged as they are), then one int -> float convert (exact:
//     |P_b| < 2^24) before the FMA;
//   * fp16: two v_mfma_f32_32x32x16_f16 over the block's 32 values.  The codes
//     (|q8| <= 127, q4 - 8 in [-8, 7]) are exact in fp16, every product is an
//     exact small integer and every partial sum stays below 2^24, so the fp32
//     result is P_b exactly, in any summation order; no convert is needed, but
//     staging widens every code to fp16.
// d4*d8 comes from one more f16 MFMA (32x32x8) used as an outer product: both
// operands are read from LDS as {scale, 0, 0, 0}, so only k = 0 adds and a
// product of two fp16 values is exact in fp32.  The per-element arithmetic
// does not depend on where a pair sits in a tile, so results are batch
// invariant.  Q8_0 and Q4_1 weights run the int8 formulation with their own
// staging (codes as they are; nibbles 0..15); the Q4_1 offset term m*d8*sum(q8)
// is added by one bf16 matrix product per pass (see offset_a_operand).
//
// Operands.  The Q8_1 activation blocks are read in place (36 bytes: fp16
// scale, fp16 sum, 32 int8 codes) and staged into LDS per pass of two blocks,
// with the weight blocks of the tile's 128 rows; the two blocks of a pass that
// belong to one row are loaded by adjacent lanes.  Tiles are double buffered
// in LDS (loads for block pair s+1 are in flight while block pair s is
// multiplied); the global loads are buffer loads whose per-lane offsets are
// fixed for a tile and whose per-pass advance is a scalar offset.  In ragged
// tiles a wave whose rows hold no pair skips its MFMA work.  A third kernel
// (namespace ws) runs the fp16 formulation warp-specialised, loader and MMA
// waves paced by LDS counters; it is kept for comparison.
//
// Fused gated activation (kFused): a tile's 128 weight rows are the gate rows
// of 64 output columns followed by their up rows; after the K loop the waves
// holding up values pass them through LDS to the waves holding the gates,
// which write act(gate) * up.  Workgroups are mapped to tiles XCD by XCD: each
// of the 8 XCDs takes a contiguous range of tiles, walked in groups of kGroupM
// M tiles with the N tiles inner, so a gathered activation tile and an expert's
// weight tiles are reused from that XCD's L2.
#include <type_traits>

#include "ftq_internal.h"

namespace ftq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kBN = 128;          // weight rows per tile
constexpr int kKB = 2;            // quantisation blocks per staged pass
constexpr int kBlockF16 = 64;     // LDS bytes of one block's 32 fp16 codes
constexpr int kRowBytes = kKB * kBlockF16;   // LDS bytes per staged row (16-byte chunks, swizzled)
constexpr int kXcds = 8;
constexpr int kGroupM = 4;
constexpr int kBufferFlags = 0x00020000;      // raw buffer resource: 32-bit data, no swizzle

// LDS row layout: 16-byte chunk c (0..7) of staged row r sits at chunk
// c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1).  Lanes reading one logical chunk
// of consecutive rows then hit 8 distinct chunks in every 8 consecutive rows
// and in every 8 rows of one parity among 16, so the fragment reads (32 rows
// per half-wave) and the stage writes (8 chunks of one row) are free of bank
// conflicts for 8 or for 16 lanes served per clock.  f depends on r % 16 only,
// so every 32-row sub-tile has the swizzle of its lane's row l32.
__device__ __forceinline__ int row_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_chunk(int r, int c) { return r * kRowBytes + ((c ^ row_swizzle(r)) << 4); }

// int8 variant: a staged row is the 2 x 32 int8 codes of a pass (64 bytes, 4
// chunks); chunk c of row r sits at chunk c ^ g(r), g(r) = gray((r >> 1) & 3)
// ^ ((r >> 3) & 1), gray(x) = x ^ (x >> 1).  Reading one logical chunk, 8
// consecutive rows then cover the 8 16-byte slots of 128 bytes and 16
// consecutive rows the 16 slots of 256 bytes; the stage writes (two chunks of
// each of 8 rows per 16 lanes) likewise.  So fragment reads and stage writes
// are free of bank conflicts for 8 or 16 lanes served per clock (the
// (r >> 1) & 3 swizzle alone is conflict-free for 8 only).
constexpr int kRowBytesI8 = kKB * 32;
__device__ __forceinline__ int row_swizzle_i8(int r) { return ((r >> 1) & 3) ^ ((r >> 2) & 1) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_chunk_i8(int r, int c) { return r * kRowBytesI8 + ((c ^ row_swizzle_i8(r)) << 4); }

// Four Q4_0 nibbles (the low or high nibbles of four bytes, already masked to
// 0..15) to the signed int8 values q - 8 in the same bytes: v + 0x78 stays
// below 0x100 in every byte (no carries), and flipping bit 7 then gives
// v - 8 modulo 256.
__device__ __forceinline__ uint32_t nibbles_minus8(uint32_t v) { return (v + 0x78787878u) ^ 0x80808080u; }

// Weight block bytes of the types the grouped path takes (GGUF layouts):
// Q4_0 {fp16 d, 16 nibble bytes}, Q4_1 {fp16 d, fp16 m, 16 nibble bytes},
// Q8_0 {fp16 d, 32 int8}.
template <int WT>
__host__ __device__ constexpr int w_bytes() { return WT == FTQ_W_Q8_0 ? 34 : WT == FTQ_W_Q4_1 ? 20 : kQ4Bytes; }

// The Q4_1 offset term m4 d8 sum(q8) of a block, as one bf16 matrix product:
// v = d8 sum(q8) is exact in fp32 (11 x 12 significant bits) and splits by
// truncation into three bf16 pieces v1 + v2 + v3 = v (8 + 8 + 8 bits); m4 (fp16)
// splits into ma + mb = m4 (8 + 3 bits).  The six products are exact in fp32,
// so the operands [v1 v1 v2 v2 v3 v3 0 0] . [ma mb ma mb ma mb 0 0] give
// v m4 up to the product's fp32 accumulation.  Packed as four words of bf16
// pairs (the upper halves of the fp32 bit patterns).
__device__ __forceinline__ uint32_t bf16_hi(float x) { return __float_as_uint(x) & 0xffff0000u; }
__device__ __forceinline__ u32x4 offset_a_operand(float v)
{
    const uint32_t b1 = bf16_hi(v);
    const float r1 = v - __uint_as_float(b1);
    const uint32_t b2 = bf16_hi(r1);
    const uint32_t b3 = bf16_hi(r1 - __uint_as_float(b2));
    return u32x4{b1 | (b1 >> 16), b2 | (b2 >> 16), b3 | (b3 >> 16), 0u};
}
__device__ __forceinline__ u32x4 offset_b_operand(float m)
{
    const uint32_t ma = bf16_hi(m);
    const uint32_t mb = bf16_hi(m - __uint_as_float(ma));
    const uint32_t w = (ma >> 16) | mb;
    return u32x4{w, w, w, 0u};
}
__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Buffer resource over `range` bytes from `base` (range: a 32-bit unsigned
// count carried in an int).  Both arguments must be wave-uniform: a resource
// the compiler thinks divergent costs a loop per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int range)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, range, kBufferFlags);
}

struct GroupedParams {
    const uint8_t* w;
    const uint8_t* a;         // Q8_1 activation rows [act rows][nb][36 B]
    float* out;
    int32_t* partials;
    const int32_t* offsets;   // [E+2]
    const int32_t* tiles;     // [E+2]
    const int32_t* sorted;
    const int4* tdesc;        // per M tile {bucket, first slot, rows, 0}
    int64_t E, N, nb, top_k, nbuckets, n_tiles_n, max_mt;
    int64_t act_div;          // activation row of pair p: p / act_div
    int32_t a_range;          // bytes of a (32-bit unsigned count; narrow variant only: below 4 GiB)
    int32_t wtile_range;      // bytes of kBN weight rows (fused: of one expert)
    int64_t half;             // fused: N/2 output columns
    int act;                  // fused: FTQ_ACT_*
};

// Waves per workgroup for BM = 128 tiles.  4 waves of 64x64 (two workgroups
// per CU, two waves per SIMD) measure fastest; 8 waves of 32x64 need 128
// VGPRs for four waves per SIMD and spill, and at one workgroup per CU they
// lose the overlap between workgroups.
constexpr int kWaves128 = 4;

template <int BM>
struct Shape {
    static constexpr int kWaves = BM == 128 ? kWaves128 : 4;
    static constexpr int kThreads = 64 * kWaves;
    // register budget: two workgroups per CU (HIP reads the second launch
    // bound as waves per SIMD)
    static constexpr int kWavesPerSimd = 2 * kWaves / 4;
    static constexpr int WM = kWaves == 8 ? 4 : (BM >= 64 ? 2 : 1);   // waves along M
    static constexpr int WN = kWaves / WM;               // waves along N
    static constexpr int SM = BM / (32 * WM);            // 32x32 sub-tiles per wave along M
    static constexpr int SN = kBN / (32 * WN);           // ... along N
    static_assert(SM >= 1 && SN >= 1, "tile shape");
};

template <int BM, bool kI8 = false, bool kOff = false>
struct Smem {
    static constexpr int RB = kI8 ? kRowBytesI8 : kRowBytes;
    // the fused epilogue exchanges BM x (kBN/2 + 4) floats through the stage
    // buffers; the int8 buffers are smaller, so they are padded up to that
    static constexpr int kStage = 2 * (BM + kBN) * RB, kExchange = BM * (kBN / 2 + 4) * 4;
    uint8_t a[2][BM * RB];
    uint8_t b[2][kBN * RB];
    uint8_t pad[kExchange > kStage ? kExchange - kStage : 16];
    uint2 as[2][kKB][BM];        // {fp16 scale bits, 0} of the A rows
    uint2 bs[2][kKB][kBN + 1];   // {fp16 scale bits, 0} of the weight rows; entry kBN stays zero
    // Q4_1: the offset product's operands per block of each A row and weight row
    u32x4 aoff[2][kKB][kOff ? BM : 1];
    u32x4 boff[2][kKB][kOff ? kBN : 1];
    int32_t row_pair[BM];
    int32_t row_tok[BM];
};

// Four packed fp16 pairs (q - 8) from one word of eight Q4_0 nibbles.  Word j of
// a block holds elements 4j..4j+3 in its low nibbles and 16+4j..16+4j+3 in its
// high nibbles; the outputs are the pairs (4j, 4j+2), (4j+1, 4j+3),
// (16+4j, 16+4j+2), (16+4j+1, 16+4j+3).  0x6400 | q is the fp16 1024 + q.
// mask = 0x000f000f and magic = 0x64006400 come in registers so that each
// mask-and-or is one instruction.
__device__ __forceinline__ void nibbles_to_f16(uint32_t x, uint32_t mask, uint32_t magic, uint32_t o[4])
{
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const uint32_t t0 = (x & mask) | magic;
    const uint32_t t1 = ((x >> 8) & mask) | magic;
    const uint32_t t2 = ((x >> 4) & mask) | magic;
    const uint32_t t3 = ((x >> 12) & mask) | magic;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, t0) + bias);
    o[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, t1) + bias);
    o[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, t2) + bias);
    o[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, t3) + bias);
}

// Two packed fp16 pairs from one word of four int8 codes: (byte 0, byte 2) and
// (byte 1, byte 3).  Each code q is offset to the byte q + 128, placed under the
// exponent byte 0x64 (the fp16 1024 + byte) and shifted back by 1152: exact.
__device__ __forceinline__ void int8_pairs_to_f16(uint32_t x, uint32_t magic, uint32_t& even, uint32_t& odd)
{
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t u = x ^ 0x80808080u;
    even = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, __builtin_amdgcn_perm(magic, u, 0x04020400u)) + bias);
    odd = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, __builtin_amdgcn_perm(magic, u, 0x04030401u)) + bias);
}

// Blocks per row, padded to whole passes.  A block past K/32 (odd K/32, last
// pass only) is read from block K/32-1 with scale 0 on both sides, so it adds
// fma(P, 0, acc) = acc exactly.
__host__ __device__ constexpr int64_t padded_blocks(int64_t nb) { return (nb + kKB - 1) / kKB * kKB; }

// ---- the tile kernel ------------------------------------------------------------

// Map a flat workgroup index to the logical tile index so that each XCD (which
// receives workgroups i with i % 8 == xcd) gets one contiguous range of tiles.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t G)
{
    const int64_t xcd = bid % kXcds, local = bid / kXcds;
    const int64_t q = G / kXcds, r = G % kXcds;
    return xcd * q + min<int64_t>(xcd, r) + local;
}

template <int BM, int VEC, bool kWide, bool kPartials, bool kFused, bool kI8, int WT = FTQ_W_Q4_0>
__global__ __launch_bounds__(Shape<BM>::kThreads, Shape<BM>::kWavesPerSimd) void moe_grouped_kernel(GroupedParams p)
{
    static_assert(WT == FTQ_W_Q4_0 || (kI8 && !kFused), "Q4_1 and Q8_0 weights: int8 block products, plain output");
    static_assert(WT != FTQ_W_Q8_0 || VEC == 4, "Q8_0 rows are read as 4-byte words (K/32 even)");
    using S = Shape<BM>;
    constexpr int kThreads = S::kThreads;
    constexpr int kWB = w_bytes<WT>();
    constexpr bool kOff = WT == FTQ_W_Q4_1 && !kPartials;   // the Q4_1 offset term
    constexpr int RB = Smem<BM, kI8>::RB;
    __shared__ __align__(16) Smem<BM, kI8, kOff> sm;

    // the wave index is uniform per wave: say so, so that what derives from it
    // (sub-tile counts, loop control) stays in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform((int32_t)(tid >> 6));
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t total_tiles = p.tiles[p.nbuckets];
    const int64_t work = total_tiles * p.n_tiles_n;
    const bool direct = (int64_t)gridDim.x >= work;   // one workgroup per tile: remap by XCD
    const int64_t nb = p.nb;
    const int64_t nbp = padded_blocks(nb);

    uint32_t nib_mask = 0x000f000fu, nib_magic = 0x64006400u;
    __asm__ volatile("" : "+v"(nib_mask), "+v"(nib_magic));
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.a, p.a_range);
    uint32_t i8_magic = 0x64646464u;
    __asm__ volatile("" : "+v"(i8_magic));

    for (int64_t w = blockIdx.x; w < work; w += gridDim.x) {
        const int64_t L = direct ? xcd_remap(w, work) : w;
        // groups of kGroupM M tiles, N tiles inner
        const int64_t grp = L / (kGroupM * p.n_tiles_n);
        const int64_t rem = L - grp * (kGroupM * p.n_tiles_n);
        const int64_t mt0 = grp * kGroupM;
        const int64_t gsz = min<int64_t>(kGroupM, total_tiles - mt0);
        const int64_t nt = rem / gsz;
        const int64_t mt = mt0 + (rem - nt * gsz);

        // bucket of this M tile: the last b with tiles[b] <= mt
        int lo = 0, hi = (int)p.nbuckets;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.tiles[mid] <= mt) lo = mid; else hi = mid;
        }
        const int64_t bucket = lo;
        const int64_t slot0 = p.offsets[bucket] + (mt - p.tiles[bucket]) * BM;
        const int rows = (int)min<int64_t>(BM, p.offsets[bucket + 1] - slot0);
        // first output column of the tile (fused: kBN/2 columns of gate and up rows)
        const int64_t n0 = nt * (kFused ? kBN / 2 : kBN);

        __syncthreads();   // the previous tile is done with LDS
        for (int m = tid; m < BM; m += kThreads) {
            const int32_t pid = m < rows ? p.sorted[slot0 + m] : 0;
            sm.row_pair[m] = pid;
            sm.row_tok[m] = (int32_t)(pid / p.act_div);
        }
        if (tid < 2 * kKB) sm.bs[tid / kKB][tid % kKB][kBN] = uint2{0u, 0u};
        __syncthreads();

        if (bucket == p.E) {   // masked pairs: zero rows
            constexpr int kCols = kFused ? kBN / 2 : kBN;
            const int64_t width = kFused ? p.half : p.N;
            for (int i = tid; i < rows * kCols; i += kThreads) {
                const int m = i / kCols, n = i - m * kCols;
                if (n0 + n >= width) continue;
                const int64_t o = (int64_t)sm.row_pair[m] * width + n0 + n;
                if constexpr (kPartials) {
                    for (int64_t b = 0; b < nb; ++b) p.partials[o * nb + b] = 0;
                } else {
                    p.out[o] = 0.0f;
                }
            }
            continue;
        }

        // ---- per-tile staging plan ------------------------------------------
        // Every global address is a per-thread offset fixed for the tile plus
        // a workgroup-uniform offset that advances by a constant per pass (the
        // scalar offset of a buffer load).  Rows past the tile (A) or past N
        // (B) read valid memory and are never stored.  A block past K/32 (odd
        // K/32, last pass only) is read from block K/32-1 on both sides with
        // scale 0, so it adds fma(P, 0, acc) = acc exactly.
        // A: one Q8_1 block (36 B: fp16 d, fp16 s, 32 int8 codes) of one row per
        // thread of the first BM * kKB threads, the two blocks of a row in
        // adjacent lanes
        static_assert(BM * kKB <= kThreads, "one activation block per thread");
        const bool a_thread = tid < BM * kKB;
        const int am = (tid / kKB) % BM, ablk = tid % kKB;
        using AOff = typename std::conditional<kWide, int64_t, uint32_t>::type;
        const AOff a_off_g = (AOff)(((int64_t)sm.row_tok[am < rows ? am : 0] * nb + ablk) * kQ8Bytes);
        int a_lds[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a_lds[j] = kI8 ? lds_chunk_i8(am, ablk * 2 + (j & 1)) : lds_chunk(am, ablk * 4 + j);
        // B: one block (18 B) of one weight row per thread of the first
        // kBN * kKB threads; bh is uniform per wave
        static_assert(kBN * kKB <= kThreads, "one weight block per thread");
        const bool b_thread = tid < kBN * kKB;
        const int bn = tid / kKB, bh = tid % kKB;   // the blocks of one row in adjacent lanes
        // uniform per tile: the tile's first weight row, or (fused) the expert's
        const uint8_t* wtile = p.w + (uniform(bucket) * p.N + (kFused ? 0 : uniform(n0))) * nb * kWB;
        const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wtile, p.wtile_range);
        uint32_t bg_off;
        if constexpr (kFused) {
            // tile row bn: gate row of column n0 + bn (bn < 64) or up row of column n0 + bn - 64
            const int64_t c = n0 + bn % (kBN / 2);
            bg_off = (uint32_t)((c < p.half ? (bn >= kBN / 2 ? p.half : 0) + c : 0) * nb * kQ4Bytes);
        } else {
            bg_off = (uint32_t)((n0 + bn < p.N ? bn : 0) * nb * kWB);
        }
        int b_lds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b_lds[i] = kI8 ? lds_chunk_i8(bn, bh * 2 + (i & 1)) : lds_chunk(bn, bh * 4 + i);

        u32x4 ra0, ra1;
        uint32_t ra2;
        bool ra_ok;
        uint32_t rb[9];
        bool rb_ok;

        auto issue = [&](int64_t kb0) {
            ra_ok = kb0 + ablk < nb;
            if (a_thread) {
                const AOff voff = ra_ok ? a_off_g : a_off_g - kQ8Bytes;
                if constexpr (kWide) {
                    typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
                    const uint8_t* abase = p.a + kb0 * kQ8Bytes + voff;
                    ra0 = *reinterpret_cast<const u32x4_a4*>(abase);
                    ra1 = *reinterpret_cast<const u32x4_a4*>(abase + 16);
                    ra2 = *reinterpret_cast<const uint32_t*>(abase + 32);
                } else {
                    const int soff = uniform((int32_t)(kb0 * kQ8Bytes));
                    ra0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, voff, soff, 0));
                    ra1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, voff + 16, soff, 0));
                    ra2 = __builtin_amdgcn_raw_buffer_load_b32(ars, voff + 32, soff, 0);
                }
            }
            // past K/32 only in the last pass of an odd K/32; uniform per wave
            rb_ok = kb0 + bh < nb;
            if (!b_thread) return;
            const int wsoff = uniform((int32_t)(kb0 * kWB));
            if constexpr (WT == FTQ_W_Q8_0) {
                // a pair of 34-byte blocks starts 4-byte aligned (K/32 even): block
                // kb0 is words 0..8 of the pair (scale in the low half of word 0,
                // codes from byte 2), block kb0+1 words 8..16 (scale in the high
                // half of word 8, codes in words 9..16).  Both lanes load two
                // 16-byte pieces and word 8.
                const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, bg_off + (bh ? 36u : 0u), wsoff, 0));
                const u32x4 y = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, bg_off + (bh ? 52u : 16u), wsoff, 0));
                rb[0] = x.x; rb[1] = x.y; rb[2] = x.z; rb[3] = x.w;
                rb[4] = y.x; rb[5] = y.y; rb[6] = y.z; rb[7] = y.w;
                rb[8] = __builtin_amdgcn_raw_buffer_load_b32(wrs, bg_off + 32u, wsoff, 0);
            } else if constexpr (WT == FTQ_W_Q4_1) {
                // 20-byte blocks: every block starts 4-byte aligned (VEC 4), else
                // ten 2-byte loads
                const uint32_t boff = bg_off + (uint32_t)((rb_ok ? bh : nb - 1 - kb0) * kWB);
                if constexpr (VEC == 4) {
                    const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, boff, wsoff, 0));
                    rb[0] = x.x; rb[1] = x.y; rb[2] = x.z; rb[3] = x.w;
                    rb[4] = __builtin_amdgcn_raw_buffer_load_b32(wrs, boff + 16, wsoff, 0);
                } else {
#pragma unroll
                    for (int i = 0; i < 5; ++i)
                        rb[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, boff + 4 * i, wsoff, 0) |
                                ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, boff + 4 * i + 2, wsoff, 0) << 16);
                }
            } else if constexpr (VEC == 4) {
                // a pair of blocks starts 4-byte aligned (K/32 even, kb0 even):
                // block kb0 is words 0..4 of the pair, block kb0+1 words 4..8
                const u32x4 w4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, bg_off + 16 * bh, wsoff, 0));
                rb[0] = w4.x; rb[1] = w4.y; rb[2] = w4.z; rb[3] = w4.w;
                rb[4] = __builtin_amdgcn_raw_buffer_load_b32(wrs, bg_off + 16 * bh + 16, wsoff, 0);
            } else {
                const uint32_t boff = bg_off + (uint32_t)((rb_ok ? bh : nb - 1 - kb0) * kQ4Bytes);
                rb[0] = __builtin_amdgcn_raw_buffer_load_b16(wrs, boff, wsoff, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    rb[1 + i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, boff + 2 + 4 * i, wsoff, 0) |
                                ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, boff + 4 + 4 * i, wsoff, 0) << 16);
            }
        };
        auto commit = [&](int buf) {
            if (a_thread) {
                const uint32_t cw[8] = {ra0.y, ra0.z, ra0.w, ra1.x, ra1.y, ra1.z, ra1.w, ra2};
                if constexpr (kI8) {
                    // the codes as they are: chunk 0 holds codes 0..15, chunk 1 codes 16..31
                    *reinterpret_cast<u32x4*>(&sm.a[buf][a_lds[0]]) = u32x4{cw[0], cw[1], cw[2], cw[3]};
                    *reinterpret_cast<u32x4*>(&sm.a[buf][a_lds[1]]) = u32x4{cw[4], cw[5], cw[6], cw[7]};
                } else {
                    // 32 int8 codes -> fp16 in the order of nibbles_to_f16: chunk j holds
                    // codes 4j..4j+3 (word j) and 16+4j..16+4j+3 (word 4+j)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t o[4];
                        int8_pairs_to_f16(cw[j], i8_magic, o[0], o[1]);
                        int8_pairs_to_f16(cw[4 + j], i8_magic, o[2], o[3]);
                        *reinterpret_cast<u32x4*>(&sm.a[buf][a_lds[j]]) = u32x4{o[0], o[1], o[2], o[3]};
                    }
                }
                sm.as[buf][ablk][am] = uint2{ra_ok ? (ra0.x & 0xffffu) : 0u, 0u};
                if constexpr (kOff) {
                    int sum = 0;
#pragma unroll
                    for (int j = 0; j < 8; ++j) sum = __builtin_amdgcn_sdot4((int)cw[j], 0x01010101, sum, false);
                    const float v = ra_ok ? half_bits_to_float(ra0.x & 0xffffu) * (float)sum : 0.0f;
                    sm.aoff[buf][ablk][am] = offset_a_operand(v);
                }
            }
            if (!b_thread) return;
            if constexpr (WT == FTQ_W_Q8_0) {
                // codes as they are: chunk 0 codes 0..15, chunk 1 codes 16..31
                const bool first = bh == 0;
                uint32_t c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) c[j] = first ? __builtin_amdgcn_alignbit(rb[j + 1], rb[j], 16) : rb[j];
                *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[0]]) = u32x4{c[0], c[1], c[2], c[3]};
                *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[1]]) = u32x4{c[4], c[5], c[6], c[7]};
                sm.bs[buf][bh][bn] = uint2{first ? (rb[0] & 0xffffu) : (rb[8] >> 16), 0u};
                return;
            } else if constexpr (WT == FTQ_W_Q4_1) {
                // codes q in 0..15 (no zero point): chunk 0 the low nibbles (elements
                // 0..15), chunk 1 the high nibbles (elements 16..31)
                u32x4 lo, hi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    lo[j] = rb[1 + j] & 0x0f0f0f0fu;
                    hi[j] = (rb[1 + j] >> 4) & 0x0f0f0f0fu;
                }
                *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[0]]) = lo;
                *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[1]]) = hi;
                sm.bs[buf][bh][bn] = uint2{rb_ok ? (rb[0] & 0xffffu) : 0u, 0u};
                if constexpr (kOff) sm.boff[buf][bh][bn] = rb_ok ? offset_b_operand(half_bits_to_float(rb[0] >> 16)) : u32x4{0u, 0u, 0u, 0u};
                return;
            }
            // weight block -> 32 fp16 values (q - 8) and its scale
            uint32_t dbits, qs[4];
            if constexpr (VEC == 4) {
                const bool first = bh == 0;
                dbits = first ? (rb[0] & 0xffffu) : (rb[0] >> 16);
                qs[0] = first ? __builtin_amdgcn_alignbit(rb[1], rb[0], 16) : rb[1];
                qs[1] = first ? __builtin_amdgcn_alignbit(rb[2], rb[1], 16) : rb[2];
                qs[2] = first ? __builtin_amdgcn_alignbit(rb[3], rb[2], 16) : rb[3];
                qs[3] = first ? __builtin_amdgcn_alignbit(rb[4], rb[3], 16) : rb[4];
            } else {
                dbits = rb[0];
                qs[0] = rb[1]; qs[1] = rb[2]; qs[2] = rb[3]; qs[3] = rb[4];
            }
            if constexpr (kI8) {
                // byte i of the nibbles holds element i (low) and i + 16 (high):
                // chunk 0 gets elements 0..15, chunk 1 elements 16..31, as q - 8
                u32x4 lo, hi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    lo[j] = nibbles_minus8(qs[j] & 0x0f0f0f0fu);
                    hi[j] = nibbles_minus8((qs[j] >> 4) & 0x0f0f0f0fu);
                }
                *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[0]]) = lo;
                *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[1]]) = hi;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t o[4];
                    nibbles_to_f16(qs[j], nib_mask, nib_magic, o);
                    *reinterpret_cast<u32x4*>(&sm.b[buf][b_lds[j]]) = u32x4{o[0], o[1], o[2], o[3]};
                }
            }
            sm.bs[buf][bh][bn] = uint2{rb_ok ? dbits : 0u, 0u};
        };

        // LDS read offsets of this lane's fragments (constant over the K loop):
        // rows of a sub-tile start at multiples of 32, so the swizzle of row r
        // is that of l32 and sub-tile and buffer offsets are immediates.
        // frag[blk][s]: this lane's chunk (block blk, piece 2*half + s)
        int frag_a[kKB][2], frag_b[kKB][2];
#pragma unroll
        for (int blk = 0; blk < kKB; ++blk)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if constexpr (kI8) {
                    // one chunk per block: the lane's half of the block's 32 codes
                    const int c = (blk * 2 + half) ^ row_swizzle_i8(l32);
                    frag_a[blk][s2] = (wm * S::SM * 32 + l32) * RB + (c << 4);
                    frag_b[blk][s2] = (wn * S::SN * 32 + l32) * RB + (c << 4);
                } else {
                    const int c = (blk * 4 + 2 * half + s2) ^ row_swizzle(l32);
                    frag_a[blk][s2] = (wm * S::SM * 32 + l32) * kRowBytes + (c << 4);
                    frag_b[blk][s2] = (wn * S::SN * 32 + l32) * kRowBytes + (c << 4);
                }
            }
        const int as_row = wm * S::SM * 32 + l32;
        int bs_row[S::SN];
#pragma unroll
        for (int j = 0; j < S::SN; ++j) bs_row[j] = half ? kBN : (wn * S::SN + j) * 32 + l32;   // upper half: zero slot

        // does any row of this wave hold a pair (uniform per wave)
        const bool wave_rows = uniform((int32_t)(wm * S::SM * 32 < rows)) != 0;

        v16f acc[S::SM][S::SN];
#pragma unroll
        for (int i = 0; i < S::SM; ++i)
#pragma unroll
            for (int j = 0; j < S::SN; ++j)
#pragma unroll
                for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.0f;

        // One staged pass, int8 codes: per sub-tile and block the exact integer
        // partial from one v_mfma_i32_32x32x32_i8, converted to fp32 (exact:
        // |P| < 2^24), then one FMA with the scale product from the f16 MFMA
        // (the outer product d8 x d4)
        auto compute_i8 = [&](int buf, int64_t kb0) {
            if (!wave_rows) return;
            v4i ai[kKB][S::SM], bi[kKB][S::SN];
            v4h as_v[kKB][S::SM], bs_v[kKB][S::SN];
#pragma unroll
            for (int blk = 0; blk < kKB; ++blk) {
#pragma unroll
                for (int ii = 0; ii < S::SM; ++ii) {
                    ai[blk][ii] = *reinterpret_cast<const v4i*>(&sm.a[buf][frag_a[blk][0] + ii * 32 * RB]);
                    as_v[blk][ii] = __builtin_bit_cast(v4h, sm.as[buf][blk][as_row + ii * 32]);
                }
#pragma unroll
                for (int jj = 0; jj < S::SN; ++jj) {
                    bi[blk][jj] = *reinterpret_cast<const v4i*>(&sm.b[buf][frag_b[blk][0] + jj * 32 * RB]);
                    bs_v[blk][jj] = __builtin_bit_cast(v4h, sm.bs[buf][blk][bs_row[jj]]);
                }
            }
            if constexpr (kPartials) {
#pragma unroll
                for (int blk = 0; blk < kKB; ++blk)
#pragma unroll
                    for (int i = 0; i < S::SM; ++i)
#pragma unroll
                        for (int j = 0; j < S::SN; ++j) {
                            const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai[blk][i], bi[blk][j], v16i{}, 0, 0, 0);
                            const int64_t n = n0 + (wn * S::SN + j) * 32 + l32;
                            const int64_t b = kb0 + blk;
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int m = (wm * S::SM + i) * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                                if (m < rows && n < p.N && b < nb)
                                    p.partials[((int64_t)sm.row_pair[m] * p.N + n) * nb + b] = P[r];
                            }
                        }
            } else {
                constexpr int kSub = S::SM * S::SN, kSteps = kKB * kSub;
                v16i P[2];
                v16f Sc[2];
                auto mm = [&](int st) {
                    const int blk = st / kSub, t = st % kSub, i = t / S::SN, j = t % S::SN;
                    P[st & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai[blk][i], bi[blk][j], v16i{}, 0, 0, 0);
                    Sc[st & 1] = __builtin_amdgcn_mfma_f32_32x32x8f16(as_v[blk][i], bs_v[blk][j], v16f{}, 0, 0, 0);
                };
                // the compiler's own schedule: forcing the next step's products
                // among this step's converts and FMAs (as the fp16 variant does)
                // measured 7 % slower here
#pragma unroll
                for (int st = 0; st < kSteps; ++st) {
                    mm(st);
                    const int t = st % kSub, i = t / S::SN, j = t % S::SN;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] = __builtin_fmaf((float)P[st & 1][r], Sc[st & 1][r], acc[i][j][r]);
                }
                if constexpr (kOff) {
                    // the Q4_1 offset terms of both blocks of the pass, added to acc
                    // by one bf16 product: lanes of the lower half carry block 0's
                    // operands, the upper half block 1's
#pragma unroll
                    for (int i = 0; i < S::SM; ++i) {
                        const v8bf ao = __builtin_bit_cast(v8bf, sm.aoff[buf][half][as_row + i * 32]);
#pragma unroll
                        for (int j = 0; j < S::SN; ++j) {
                            const v8bf bo = __builtin_bit_cast(v8bf, sm.boff[buf][half][(wn * S::SN + j) * 32 + l32]);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bo, acc[i][j], 0, 0, 0);
                        }
                    }
                }
            }
        };
        // One staged pass: kKB blocks from LDS buffer `buf`
        auto compute = [&](int buf, int64_t kb0) {
            if constexpr (kI8) {
                compute_i8(buf, kb0);
                return;
            }
            if (!wave_rows) return;
            v8h alo[kKB][S::SM], ahi[kKB][S::SM], blo[kKB][S::SN], bhi[kKB][S::SN];
            v4h as_v[kKB][S::SM], bs_v[kKB][S::SN];
#pragma unroll
            for (int blk = 0; blk < kKB; ++blk) {
#pragma unroll
                for (int ii = 0; ii < S::SM; ++ii) {
                    alo[blk][ii] = *reinterpret_cast<const v8h*>(&sm.a[buf][frag_a[blk][0] + ii * 32 * kRowBytes]);
                    ahi[blk][ii] = *reinterpret_cast<const v8h*>(&sm.a[buf][frag_a[blk][1] + ii * 32 * kRowBytes]);
                    as_v[blk][ii] = __builtin_bit_cast(v4h, sm.as[buf][blk][as_row + ii * 32]);
                }
#pragma unroll
                for (int jj = 0; jj < S::SN; ++jj) {
                    blo[blk][jj] = *reinterpret_cast<const v8h*>(&sm.b[buf][frag_b[blk][0] + jj * 32 * kRowBytes]);
                    bhi[blk][jj] = *reinterpret_cast<const v8h*>(&sm.b[buf][frag_b[blk][1] + jj * 32 * kRowBytes]);
                    bs_v[blk][jj] = __builtin_bit_cast(v4h, sm.bs[buf][blk][bs_row[jj]]);
                }
            }
            if constexpr (kPartials) {
#pragma unroll
                for (int blk = 0; blk < kKB; ++blk)
#pragma unroll
                    for (int i = 0; i < S::SM; ++i)
#pragma unroll
                        for (int j = 0; j < S::SN; ++j) {
                            v16f P = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[blk][i], blo[blk][j], v16f{}, 0, 0, 0);
                            P = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[blk][i], bhi[blk][j], P, 0, 0, 0);
                            const int64_t n = n0 + (wn * S::SN + j) * 32 + l32;
                            const int64_t b = kb0 + blk;
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int m = (wm * S::SM + i) * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                                if (m < rows && n < p.N && b < nb)
                                    p.partials[((int64_t)sm.row_pair[m] * p.N + n) * nb + b] = (int32_t)P[r];
                            }
                        }
            } else {
                // products of step s+1 are issued before the FMAs of step s, so
                // the matrix cores and the vector ALUs work at the same time
                constexpr int kSub = S::SM * S::SN, kSteps = kKB * kSub;
                v16f P[2], Sc[2];
                auto mm = [&](int st) {
                    const int blk = st / kSub, t = st % kSub, i = t / S::SN, j = t % S::SN;
                    v16f q = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[blk][i], blo[blk][j], v16f{}, 0, 0, 0);
                    P[st & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[blk][i], bhi[blk][j], q, 0, 0, 0);
                    Sc[st & 1] = __builtin_amdgcn_mfma_f32_32x32x8f16(as_v[blk][i], bs_v[blk][j], v16f{}, 0, 0, 0);
                };
                mm(0);
#pragma unroll
                for (int st = 0; st < kSteps; ++st) {
                    if (st + 1 < kSteps) mm(st + 1);
                    const int t = st % kSub, i = t / S::SN, j = t % S::SN;
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(P[st & 1][r], Sc[st & 1][r], acc[i][j][r]);
#if 1
                    if (st + 1 < kSteps) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                    }
#endif
                }
            }
        };
        // ---- K loop: double-buffered, unrolled by two so buffers are constants
        const int64_t nstages = nbp / kKB;
        issue(0);
        commit(0);
        __syncthreads();
        for (int64_t s = 0; s < nstages; s += 2) {
            if (s + 1 < nstages) issue((s + 1) * kKB);
            compute(0, s * kKB);
            if (s + 1 < nstages) commit(1);
            __syncthreads();
            if (s + 1 >= nstages) break;
            if (s + 2 < nstages) issue((s + 2) * kKB);
            compute(1, (s + 1) * kKB);
            if (s + 2 < nstages) commit(0);
            __syncthreads();
        }

        if constexpr (kFused) {
            // tile rows (sub-tile column groups) below kBN/2 are gates, the rest
            // the up rows of the same columns: exchange through LDS, which the
            // K loop no longer uses (its last barrier has passed)
            constexpr int kXPitch = kBN / 2 + 4;   // floats per exchanged row
            static_assert(BM * kXPitch * 4 <= (int)(sizeof(sm.a) + sizeof(sm.b) + sizeof(sm.pad)), "exchange fits the stage buffers");
            float* xch = reinterpret_cast<float*>(&sm.a[0][0]);
            int l32e = l32, halfe = half;
            __asm__ volatile("" : "+v"(l32e), "+v"(halfe));
#pragma unroll
            for (int i = 0; i < S::SM; ++i)
#pragma unroll
                for (int j = 0; j < S::SN; ++j) {
                    const int R = (wn * S::SN + j) * 32;   // first tile row of the sub-tile (uniform)
                    if (R >= kBN / 2) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = (wm * S::SM + i) * 32 + 8 * (r / 4) + 4 * halfe + (r % 4);
                            xch[m * kXPitch + R - kBN / 2 + l32e] = acc[i][j][r];
                        }
                    }
                }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < S::SM; ++i)
#pragma unroll
                for (int j = 0; j < S::SN; ++j) {
                    const int R = (wn * S::SN + j) * 32;
                    if (R < kBN / 2) {
                        const int64_t c = n0 + R + l32e;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = (wm * S::SM + i) * 32 + 8 * (r / 4) + 4 * halfe + (r % 4);
                            if (m < rows && c < p.half)
                                __builtin_nontemporal_store(gated_act(p.act, acc[i][j][r]) * xch[m * kXPitch + R + l32e],
                                                            &p.out[(int64_t)sm.row_pair[m] * p.half + c]);
                        }
                    }
                }
        } else if constexpr (!kPartials) {
            // row and column of this lane's outputs, made opaque here so that
            // the compiler does not compute them before the K loop and keep them
            // live through it
            int l32e = l32, halfe = half;
            __asm__ volatile("" : "+v"(l32e), "+v"(halfe));
#pragma unroll
            for (int i = 0; i < S::SM; ++i) {
#pragma unroll
                for (int j = 0; j < S::SN; ++j) {
                    const int64_t n = n0 + (wn * S::SN + j) * 32 + l32e;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = (wm * S::SM + i) * 32 + 8 * (r / 4) + 4 * halfe + (r % 4);
                        if (m < rows && n < p.N)
                            __builtin_nontemporal_store(acc[i][j][r], &p.out[(int64_t)sm.row_pair[m] * p.N + n]);
                    }
                }
            }
        }
    }
}

// ---- the warp-specialised tile kernel (128-row tiles) ---------------------------
//
// One workgroup of 8 waves per CU, persistent over its share of the tiles.
// Waves 4-7 (producers, one per SIMD) load the Q8_1 and Q4_0 blocks of a
// stage (two quantisation blocks of the tile), widen them to fp16 in the
// layout above and write them into a ring of kRing stages in LDS.  Waves 0-3
// (consumers, one per SIMD) read their fragments from the ring and run the
// matrix products and the scale-accumulate.  The two sides are paced by
// per-stage counters in LDS instead of workgroup barriers: a producer waits
// until all consumers have released the slot it is about to overwrite, a
// consumer until all producers have filled the stage it is about to read.  So
// on every SIMD one wave issues matrix products while the other converts and
// stages, and the loads of the next kLoadAhead stages are always in flight.
// Every wait is bounded (kSpinLimit polls): a broken invariant ends in wrong
// results, never in a hung GPU.
//
// Consumer c holds a 64 x 64 part of the tile: M sub-tiles i = 0, 1 cover tile
// rows (2i + c/2) * 32 .. +31 (interleaved, so that a ragged tile's rows are
// shared by both consumer pairs), N sub-tiles j = 0, 1 cover weight rows
// (c%2) * 64 + j * 32 .. +31.  With the fused activation sub-tile j = 0 holds
// the gate rows and j = 1 the up rows of the same 32 output columns, so gate
// and up of an output meet in one lane's registers.  Within a stage the
// products of step s + 1 are issued among the scale-accumulates of step s, in
// a fixed order the compiler is not allowed to change, and the fragments of
// the next block are read while the current one is multiplied.
namespace ws {

constexpr int kThreads = 512;            // 4 consumer + 4 producer waves
constexpr int kBM = 128;
constexpr int kRing = 4;                 // stages in LDS (kKB blocks each)
constexpr int kLoadAhead = kRing;        // stages of loads in flight per producer thread (divides or is a multiple of kRing)
constexpr int kTabs = kRing + kLoadAhead + 2;   // see the producer's table writes
constexpr int kConsumers = 4;
constexpr int kProducers = 4;
constexpr int kSpinLimit = 1 << 16;     // about 5 ms per wait at most

struct Smem {
    uint8_t a[kRing][kBM * kRowBytes];
    uint8_t b[kRing][kBN * kRowBytes];
    uint2 as[kRing][kKB][kBM];           // {fp16 scale bits, 0} of the A rows
    uint2 bs[kRing][kKB][kBN + 1];       // ... of the weight rows; entry kBN stays zero
    int32_t pid[kTabs][kBM];             // pair of each tile row, per tile in flight
    int32_t desc[kTabs][4];              // rows, first slot, first column of the tile
    int32_t ready[kRing];                // producer waves that have filled the slot, in total
    int32_t empty[kRing];                // consumer waves that have released the slot, in total
};

// Wait until *ctr >= target (LDS, written by other waves of the workgroup).
__device__ __forceinline__ void wait_at_least(int32_t* ctr, int32_t target)
{
    for (int spins = 0; spins < kSpinLimit; ++spins) {
        const int32_t v = uniform(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __asm__ volatile("" ::: "memory");   // the stage's LDS accesses stay after the wait
}

// Count this wave in: its LDS reads (consumer) or writes (producer) of the
// stage have completed before the counter moves.
__device__ __forceinline__ void arrive(int32_t* ctr, int lane)
{
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The tiles of this workgroup, in order: each XCD takes a contiguous range of
// the work items (so an expert's weights and a group's activation rows are
// shared in that XCD's L2) and its workgroups take the items of the range in
// turn.
struct WorkIter {
    int64_t cur, end, step;
    __device__ __forceinline__ void init(int64_t work)
    {
        const int64_t G = gridDim.x;
        if (G >= kXcds && G % kXcds == 0) {
            const int64_t x = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
            cur = x * work / kXcds + li;
            end = (x + 1) * work / kXcds;
            step = G / kXcds;
        } else {
            cur = blockIdx.x;
            end = work;
            step = G;
        }
    }
};

// Logical work item -> (M tile, N tile): groups of kGroupM M tiles, N tiles inner.
__device__ __forceinline__ void item_tiles(int64_t L, int64_t total_tiles, int64_t ntn, int64_t& mt, int64_t& nt)
{
    const uint32_t per = (uint32_t)(kGroupM * ntn);
    const uint32_t Lu = (uint32_t)L;   // work < 2^31 (checked on the host)
    const uint32_t grp = Lu / per, rem = Lu - grp * per;
    const uint32_t mt0 = grp * kGroupM;
    const uint32_t gsz = (uint32_t)min<int64_t>(kGroupM, total_tiles - mt0);
    const uint32_t n = rem / gsz;
    nt = n;
    mt = mt0 + (rem - n * gsz);
}

struct TileInfo {
    int64_t bucket, slot0, n0;
    int rows;
};

__device__ __forceinline__ TileInfo tile_info(const GroupedParams& p, int64_t mt, int64_t nt, int64_t col_tile)
{
    int lo = 0, hi = (int)p.nbuckets;   // the last bucket b with tiles[b] <= mt
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.tiles[mid] <= mt) lo = mid; else hi = mid;
    }
    TileInfo t;
    t.bucket = lo;
    t.slot0 = p.offsets[lo] + (mt - p.tiles[lo]) * kBM;
    t.rows = (int)min<int64_t>(kBM, p.offsets[lo + 1] - t.slot0);
    t.n0 = nt * col_tile;
    return t;
}

// Weight row that tile row bn reads: the plain tile's row n0 + bn (relative to
// the tile base), or (fused) the gate / up row of output column
// n0 + (bn/64)*32 + bn%32 relative to the expert's first row.  Rows past the
// matrix read a valid row and are never stored.
template <bool kFused>
__device__ __forceinline__ uint32_t weight_row_offset(const GroupedParams& p, int64_t n0, int bn)
{
    if constexpr (kFused) {
        const int64_t c = n0 + (bn / 64) * 32 + bn % 32;
        const int64_t row = c < p.half ? ((bn / 32) % 2 ? p.half : 0) + c : 0;
        return (uint32_t)(row * p.nb * kQ4Bytes);
    } else {
        return (uint32_t)((n0 + bn < p.N ? bn : 0) * p.nb * kQ4Bytes);
    }
}

template <int VEC, bool kWide, bool kPartials, bool kFused>
__global__ __launch_bounds__(kThreads, 2) void moe_grouped_ws_kernel(GroupedParams p)
{
    __shared__ __align__(16) Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform((int32_t)(tid >> 6));
    const int64_t nb = p.nb;
    const int64_t nstages = padded_blocks(nb) / kKB;
    const int64_t real_tiles = p.tiles[p.E];          // tiles of buckets 0..E-1; the masked bucket's follow
    const int64_t total_tiles = p.tiles[p.nbuckets];
    const int64_t work = total_tiles * p.n_tiles_n;
    constexpr int64_t kColTile = kFused ? kBN / 2 : kBN;

    for (int i = tid; i < kRing; i += kThreads) { sm.ready[i] = 0; sm.empty[i] = 0; }
    for (int i = tid; i < kRing * kKB; i += kThreads) sm.bs[i / kKB][i % kKB][kBN] = uint2{0u, 0u};
    __syncthreads();   // the only workgroup barrier: the roles never meet again

    if (wave >= kConsumers) {
        // ================================ producers ================================
        const int pt = tid - kConsumers * 64;          // 0..255
        const int am = pt / kKB, ablk = pt % kKB;      // A: tile row am, block ablk of a stage
        const int bn = pt / kKB, bh = pt % kKB;        // B: tile row bn, block bh
        uint32_t nib_mask = 0x000f000fu, nib_magic = 0x64006400u, i8_magic = 0x64646464u;
        __asm__ volatile("" : "+v"(nib_mask), "+v"(nib_magic), "+v"(i8_magic));
        const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.a, p.a_range);
        using AOff = typename std::conditional<kWide, int64_t, uint32_t>::type;

        // Load cursor: the stage whose loads are issued next.  Entering a tile
        // waits on no memory: the descriptor of the tile after next and the
        // row pairs of the next tile are loaded one tile ahead (vector loads,
        // so that the counter updates' LDS waits do not wait for them).
        WorkIter li;
        li.init(work);
        auto find_real = [&](int64_t c) -> int64_t {   // the first real tile's item at or after c
            for (; c < li.end; c += li.step) {
                int64_t mt, nt;
                item_tiles(c, total_tiles, p.n_tiles_n, mt, nt);
                if (mt < real_tiles) break;
            }
            return c;
        };
        const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.tdesc, (int32_t)(uint32_t)min<int64_t>(16 * total_tiles, UINT32_MAX));
        const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.sorted, (int32_t)(uint32_t)min<int64_t>(4 * (int64_t)p.offsets[p.nbuckets], UINT32_MAX));
        auto load_desc = [&](int64_t item) -> int4 {
            if (item >= li.end) return int4{0, 0, 0, 0};
            int64_t mt, nt;
            item_tiles(item, total_tiles, p.n_tiles_n, mt, nt);
            return __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(drs, (uint32_t)(mt * 16), 0, 0));
        };
        auto load_pid = [&](int4 d) -> int32_t {   // this thread's row pair of the tile with descriptor d
            const int32_t sl = uniform(d.y), rw = uniform(d.z);
            return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)(4 * (sl + (am < rw ? am : 0))), 0, 0);
        };
        int64_t nx1 = find_real(li.cur);           // next tile to enter
        int4 nx1_d = load_desc(nx1);
        int32_t nx1_pid = nx1 < li.end ? load_pid(nx1_d) : 0;
        int64_t nx2 = nx1 < li.end ? find_real(nx1 + li.step) : li.end;
        int4 nx2_d = load_desc(nx2);
        int64_t l_kb0 = 0;
        bool l_valid = false;
        int64_t l_rseq = 0;                      // real tiles entered so far
        AOff a_off_g = 0;
        uint32_t bg_off = 0;
        __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.w, 0);
        auto l_enter = [&]() {
            l_valid = nx1 < li.end;
            if (!l_valid) return;
            int64_t mt, nt;
            item_tiles(nx1, total_tiles, p.n_tiles_n, mt, nt);
            const int64_t bucket = uniform(nx1_d.x), slot0 = uniform(nx1_d.y);
            const int rows = uniform(nx1_d.z);
            const int64_t n0 = nt * kColTile;
            const int32_t pid = nx1_pid;
            const int32_t tok = (int32_t)((uint32_t)pid / (uint32_t)p.act_div);
            a_off_g = (AOff)(((int64_t)tok * nb + ablk) * kQ8Bytes);
            const uint8_t* wtile = p.w + (bucket * p.N + (kFused ? 0 : n0)) * nb * kQ4Bytes;
            wrs = make_rsrc(wtile, p.wtile_range);
            bg_off = weight_row_offset<kFused>(p, n0, bn);
            const int tab = (int)(l_rseq % kTabs);
            if (ablk == 0) sm.pid[tab][am] = pid;
            if (pt == 0) {
                sm.desc[tab][0] = rows;
                sm.desc[tab][1] = (int32_t)slot0;
                sm.desc[tab][2] = (int32_t)n0;
            }
            ++l_rseq;
            l_kb0 = 0;
            // move the lookahead on
            nx1 = nx2;
            nx1_d = nx2_d;
            if (nx1 < li.end) nx1_pid = load_pid(nx1_d);
            nx2 = nx1 < li.end ? find_real(nx1 + li.step) : li.end;
            nx2_d = load_desc(nx2);
        };
        auto l_advance = [&]() {
            l_kb0 += kKB;
            if (l_kb0 >= kKB * nstages) l_enter();
        };

        u32x4 ra0[kLoadAhead], ra1[kLoadAhead];
        uint32_t ra2[kLoadAhead], rb[kLoadAhead][5];
        auto issue = [&](int set) {
            const int64_t kb0 = l_kb0;
            const bool ok = kb0 + ablk < nb;
            const AOff voff = ok ? a_off_g : a_off_g - kQ8Bytes;
            if constexpr (kWide) {
                typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
                const uint8_t* abase = p.a + kb0 * kQ8Bytes + voff;
                ra0[set] = *reinterpret_cast<const u32x4_a4*>(abase);
                ra1[set] = *reinterpret_cast<const u32x4_a4*>(abase + 16);
                ra2[set] = *reinterpret_cast<const uint32_t*>(abase + 32);
            } else {
                const int soff = uniform((int32_t)(kb0 * kQ8Bytes));
                ra0[set] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, voff, soff, 0));
                ra1[set] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, voff + 16, soff, 0));
                ra2[set] = __builtin_amdgcn_raw_buffer_load_b32(ars, voff + 32, soff, 0);
            }
            const bool bok = kb0 + bh < nb;
            const int wsoff = uniform((int32_t)(kb0 * kQ4Bytes));
            if constexpr (VEC == 4) {
                const u32x4 w4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, bg_off + 16 * bh, wsoff, 0));
                rb[set][0] = w4.x; rb[set][1] = w4.y; rb[set][2] = w4.z; rb[set][3] = w4.w;
                rb[set][4] = __builtin_amdgcn_raw_buffer_load_b32(wrs, bg_off + 16 * bh + 16, wsoff, 0);
            } else {
                const uint32_t boff = bg_off + (uint32_t)((bok ? bh : nb - 1 - kb0) * kQ4Bytes);
                rb[set][0] = __builtin_amdgcn_raw_buffer_load_b16(wrs, boff, wsoff, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    rb[set][1 + i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, boff + 2 + 4 * i, wsoff, 0) |
                                     ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wrs, boff + 4 + 4 * i, wsoff, 0) << 16);
            }
        };

        // LDS write offsets of this thread (within a slot)
        int a_lds[4], b_lds[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a_lds[j] = lds_chunk(am, ablk * 4 + j);
            b_lds[j] = lds_chunk(bn, bh * 4 + j);
        }
        auto commit = [&](int set, int slot, int64_t kb0) {
            const bool ok = kb0 + ablk < nb;
            const uint32_t cw[8] = {ra0[set].y, ra0[set].z, ra0[set].w, ra1[set].x, ra1[set].y, ra1[set].z, ra1[set].w, ra2[set]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t o[4];
                int8_pairs_to_f16(cw[j], i8_magic, o[0], o[1]);
                int8_pairs_to_f16(cw[4 + j], i8_magic, o[2], o[3]);
                *reinterpret_cast<u32x4*>(&sm.a[slot][a_lds[j]]) = u32x4{o[0], o[1], o[2], o[3]};
            }
            sm.as[slot][ablk][am] = uint2{ok ? (ra0[set].x & 0xffffu) : 0u, 0u};
            const bool bok = kb0 + bh < nb;
            uint32_t dbits, qs[4];
            if constexpr (VEC == 4) {
                const bool first = bh == 0;
                dbits = first ? (rb[set][0] & 0xffffu) : (rb[set][0] >> 16);
                qs[0] = first ? __builtin_amdgcn_alignbit(rb[set][1], rb[set][0], 16) : rb[set][1];
                qs[1] = first ? __builtin_amdgcn_alignbit(rb[set][2], rb[set][1], 16) : rb[set][2];
                qs[2] = first ? __builtin_amdgcn_alignbit(rb[set][3], rb[set][2], 16) : rb[set][3];
                qs[3] = first ? __builtin_amdgcn_alignbit(rb[set][4], rb[set][3], 16) : rb[set][4];
            } else {
                dbits = rb[set][0];
                qs[0] = rb[set][1]; qs[1] = rb[set][2]; qs[2] = rb[set][3]; qs[3] = rb[set][4];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t o[4];
                nibbles_to_f16(qs[j], nib_mask, nib_magic, o);
                *reinterpret_cast<u32x4*>(&sm.b[slot][b_lds[j]]) = u32x4{o[0], o[1], o[2], o[3]};
            }
            sm.bs[slot][bh][bn] = uint2{bok ? dbits : 0u, 0u};
        };

        // commit cursor: only the block index of the stage matters to a commit
        WorkIter ci;
        ci.init(work);
        bool c_valid;
        auto c_enter = [&]() {
            for (; ci.cur < ci.end; ci.cur += ci.step) {
                int64_t mt, nt;
                item_tiles(ci.cur, total_tiles, p.n_tiles_n, mt, nt);
                if (mt < real_tiles) break;
            }
            c_valid = ci.cur < ci.end;
        };
        int64_t c_kb0 = 0;

        l_enter();
        c_enter();
#pragma unroll
        for (int s = 0; s < kLoadAhead; ++s) {
            if (l_valid) {
                issue(s);
                l_advance();
            }
        }
        // unrolled so that the slot (u % kRing) and the load set (u % kLoadAhead)
        // are constants
        constexpr int kUnroll = kRing > kLoadAhead ? kRing : kLoadAhead;
        static_assert(kUnroll % kRing == 0 && kUnroll % kLoadAhead == 0, "ring and load depth divide the unroll");
        for (int64_t g = 0; c_valid; g += kUnroll) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (!c_valid) break;
                const int slot = u % kRing, set = u % kLoadAhead;
                const int64_t use = (g + u) / kRing;
                wait_at_least(&sm.empty[slot], (int32_t)(kConsumers * use));
                commit(set, slot, c_kb0);
                arrive(&sm.ready[slot], lane);
                if (l_valid) {
                    issue(set);
                    l_advance();
                }
                c_kb0 += kKB;
                if (c_kb0 >= kKB * nstages) {
                    c_kb0 = 0;
                    ci.cur += ci.step;
                    c_enter();
                }
            }
        }
        return;
    }

    // ================================== consumers ==================================
    const int wm = wave / 2, wn = wave % 2;
    const int half = lane >> 5, l32 = lane & 31;
    // per-lane LDS offsets within a stage slot; M sub-tile i adds i * 64 rows and
    // N sub-tile j adds j * 32 rows (immediates)
    const int sw = row_swizzle(l32);
    int fa[kKB][2], fb[kKB][2];
#pragma unroll
    for (int blk = 0; blk < kKB; ++blk)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int c = (blk * 4 + 2 * half + s2) ^ sw;
            fa[blk][s2] = (wm * 32 + l32) * kRowBytes + (c << 4);
            fb[blk][s2] = (wn * 64 + l32) * kRowBytes + (c << 4);
        }
    const int as_row = wm * 32 + l32;
    const int bs_row0 = half ? kBN : wn * 64 + l32;
    const int bs_row1 = half ? kBN : wn * 64 + 32 + l32;

    // One fragment set: the pieces of block q are reloaded with block q+1's as
    // soon as their last product of block q has been issued.
    v8h Alo[2], Ahi[2], Blo[2], Bhi[2];
    v4h AS[2], BS[2];
    auto load_a = [&](int slot, int blk, int i) __attribute__((always_inline)) {
        Alo[i] = *reinterpret_cast<const v8h*>(&sm.a[slot][fa[blk][0] + i * 64 * kRowBytes]);
        Ahi[i] = *reinterpret_cast<const v8h*>(&sm.a[slot][fa[blk][1] + i * 64 * kRowBytes]);
        AS[i] = __builtin_bit_cast(v4h, sm.as[slot][blk][as_row + i * 64]);
    };
    auto load_b = [&](int slot, int blk, int j) __attribute__((always_inline)) {
        Blo[j] = *reinterpret_cast<const v8h*>(&sm.b[slot][fb[blk][0] + j * 32 * kRowBytes]);
        Bhi[j] = *reinterpret_cast<const v8h*>(&sm.b[slot][fb[blk][1] + j * 32 * kRowBytes]);
        BS[j] = __builtin_bit_cast(v4h, sm.bs[slot][blk][j ? bs_row1 : bs_row0]);
    };

    v16f acc[2][2];
    WorkIter wi;
    wi.init(work);
    int64_t g = 0;       // stages consumed so far (all tiles)
    int64_t rseq = 0;    // real tiles consumed so far
    for (; wi.cur < wi.end; wi.cur += wi.step) {
        int64_t mt, nt;
        item_tiles(wi.cur, total_tiles, p.n_tiles_n, mt, nt);
        if (mt >= real_tiles) {
            // masked pairs (ids outside [0, E)): zero rows, read straight from the pair list
            const int64_t E = p.E;
            const int64_t slot0 = p.offsets[E] + (mt - p.tiles[E]) * kBM;
            const int rows = (int)min<int64_t>(kBM, p.offsets[E + 1] - slot0);
            const int64_t n0 = nt * kColTile;
            const int64_t width = kFused ? p.half : p.N;
            for (int i = tid; i < rows * kColTile; i += kConsumers * 64) {
                const int m = i / (int)kColTile, n = i - m * (int)kColTile;
                if (n0 + n >= width) continue;
                const int64_t o = (int64_t)p.sorted[slot0 + m] * width + n0 + n;
                if constexpr (kPartials) {
                    for (int64_t b = 0; b < nb; ++b) p.partials[o * nb + b] = 0;
                } else {
                    p.out[o] = 0.0f;
                }
            }
            continue;
        }
        const int tab = (int)(rseq % kTabs);
        ++rseq;
        // the first stage of the tile is filled (and with it the tile's tables)
        wait_at_least(&sm.ready[g % kRing], (int32_t)(kProducers * (g / kRing + 1)));
        const int rows = uniform(sm.desc[tab][0]);
        const int64_t n0 = uniform(sm.desc[tab][2]);
        // live M sub-tiles of this consumer: i with (2i + wm) * 32 < rows
        const int SML = (wm * 32 < rows ? 1 : 0) + (64 + wm * 32 < rows ? 1 : 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        if (SML == 0 || kPartials) {
            // nothing to multiply (no live rows), or the checking variant
            for (int64_t s = 0; s < nstages; ++s, ++g) {
                const int slot = (int)(g % kRing);
                wait_at_least(&sm.ready[slot], (int32_t)(kProducers * (g / kRing + 1)));
                if constexpr (kPartials) {
#pragma unroll
                    for (int blk = 0; blk < kKB; ++blk) {
                        const int64_t b = s * kKB + blk;
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            if (i >= SML) continue;
                            load_a(slot, blk, i);
#pragma unroll
                            for (int j = 0; j < 2; ++j) {
                                load_b(slot, blk, j);
                                v16f P = __builtin_amdgcn_mfma_f32_32x32x16_f16(Alo[i], Blo[j], v16f{}, 0, 0, 0);
                                P = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ahi[i], Bhi[j], P, 0, 0, 0);
                                const int64_t n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int m = (2 * i + wm) * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                                    if (m < rows && n < p.N && b < nb)
                                        p.partials[((int64_t)sm.pid[tab][m] * p.N + n) * nb + b] = (int32_t)P[r];
                                }
                            }
                        }
                    }
                }
                arrive(&sm.empty[slot], lane);
            }
        } else {
            auto run = [&](auto sml_c) __attribute__((always_inline)) {
                constexpr int SM = decltype(sml_c)::value;
                constexpr int kSub = SM * 2;   // steps per block: (i, j) = (t / 2, t % 2)
                v16f P[2], Sc[2];
                auto fmas = [&](int t, int r0, int r1) __attribute__((always_inline)) {
                    const int i = t / 2, j = t % 2;
#pragma unroll
                    for (int r = r0; r < r1; ++r) acc[i][j][r] = __builtin_fmaf(P[t & 1][r], Sc[t & 1][r], acc[i][j][r]);
                };
                // step t of a block: the products of step nt (of this block, or
                // step 0 of the next block) interleaved with step t's
                // scale-accumulate, in this order:
                //   P1(nt) 5 FMA(t)  P2(nt) 5 FMA(t)  S(nt) 6 FMA(t)
                auto step = [&](int t, bool issue, int ntt) __attribute__((always_inline)) {
                    const int i = ntt / 2, j = ntt % 2, b = ntt & 1;
                    if (issue) P[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Alo[i], Blo[j], v16f{}, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    fmas(t, 0, 5);
                    __builtin_amdgcn_sched_barrier(0);
                    if (issue) P[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ahi[i], Bhi[j], P[b], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    fmas(t, 5, 10);
                    __builtin_amdgcn_sched_barrier(0);
                    if (issue) Sc[b] = __builtin_amdgcn_mfma_f32_32x32x8f16(AS[i], BS[j], v16f{}, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    fmas(t, 10, 16);
                    __builtin_amdgcn_sched_barrier(0);
                };
                // one block: kNext says whether another block of the tile follows
                // (in slot nslot, block nblk); its pieces are reloaded as this
                // block's last products that use them are issued
                auto block = [&](auto next_c, int nslot, int nblk) __attribute__((always_inline)) {
                    constexpr bool kNext = decltype(next_c)::value;
#pragma unroll
                    for (int t = 0; t < kSub; ++t) {
                        if (t + 1 < kSub) step(t, true, t + 1);
                        else step(t, kNext, 0);
                        if constexpr (kNext) {
                            if (t == 0) {
                                load_a(nslot, nblk, 0);   // last used by step 1's products
                                if (SM == 1) { load_b(nslot, nblk, 0); load_b(nslot, nblk, 1); }
                            }
                            if (SM == 2 && t == 1) load_b(nslot, nblk, 0);
                            if (SM == 2 && t == 2) { load_a(nslot, nblk, 1); load_b(nslot, nblk, 1); }
                        }
                    }
                };
                // prologue: block 0 of the tile's first stage, and its first products
                {
                    const int slot = (int)(g % kRing);
#pragma unroll
                    for (int i = 0; i < SM; ++i) load_a(slot, 0, i);
                    load_b(slot, 0, 0);
                    load_b(slot, 0, 1);
                    P[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Alo[0], Blo[0], v16f{}, 0, 0, 0);
                    P[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ahi[0], Bhi[0], P[0], 0, 0, 0);
                    Sc[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(AS[0], BS[0], v16f{}, 0, 0, 0);
                }
                // The wait for the next stage comes first, so that the stage's
                // steps are one straight run of code that nothing is moved
                // across (its pieces are read during this stage's block 1).
                for (int64_t s = 0; s + 1 < nstages; ++s) {
                    const int slot = (int)(g % kRing), nslot = (int)((g + 1) % kRing);
                    wait_at_least(&sm.ready[nslot], (int32_t)(kProducers * ((g + 1) / kRing + 1)));
                    block(std::true_type{}, slot, 1);
                    block(std::true_type{}, nslot, 0);
                    arrive(&sm.empty[slot], lane);
                    ++g;
                }
                {
                    const int slot = (int)(g % kRing);
                    block(std::true_type{}, slot, 1);
                    block(std::false_type{}, slot, 0);
                    arrive(&sm.empty[slot], lane);
                    ++g;
                }
            };
            if (SML == 2) run(std::integral_constant<int, 2>{});
            else run(std::integral_constant<int, 1>{});
        }

        if constexpr (!kPartials) {
            // epilogue: rows of tile row m = (2i + wm) * 32 + 8 (r/4) + 4 half + r%4
            int l32e = l32, halfe = half;
            __asm__ volatile("" : "+v"(l32e), "+v"(halfe));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (i >= SML) continue;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int mb = (2 * i + wm) * 32 + 8 * q4 + 4 * halfe;
                    const int4 pids = *reinterpret_cast<const int4*>(&sm.pid[tab][mb]);
                    const int32_t pv[4] = {pids.x, pids.y, pids.z, pids.w};
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int m = mb + r4, r = 4 * q4 + r4;
                        if (m >= rows) continue;
                        if constexpr (kFused) {
                            const int64_t c = n0 + wn * 32 + l32e;
                            if (c < p.half)
                                __builtin_nontemporal_store(gated_act(p.act, acc[i][0][r]) * acc[i][1][r],
                                                            &p.out[(int64_t)pv[r4] * p.half + c]);
                        } else {
#pragma unroll
                            for (int j = 0; j < 2; ++j) {
                                const int64_t n = n0 + wn * 64 + j * 32 + l32e;
                                if (n < p.N) __builtin_nontemporal_store(acc[i][j][r], &p.out[(int64_t)pv[r4] * p.N + n]);
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace ws

template <int BM, bool kPartials, bool kFused, bool kI8, int WT = FTQ_W_Q4_0>
int launch_grouped_v(int vec, bool wide, const GroupedParams& gp, int64_t grid, hipStream_t s)
{
    constexpr int kT = Shape<BM>::kThreads;
    if (vec == 4) {
        return wide ? launch("moe_grouped_kernel<4,wide>", moe_grouped_kernel<BM, 4, true, kPartials, kFused, kI8, WT>, grid, kT, 0, s, gp)
                    : launch("moe_grouped_kernel<4>", moe_grouped_kernel<BM, 4, false, kPartials, kFused, kI8, WT>, grid, kT, 0, s, gp);
    }
    if constexpr (WT == FTQ_W_Q8_0) {
        set_error("Q8_0 weights on the grouped path need K/32 even and 4-byte aligned weights");
        return FTQ_ERR_UNSUPPORTED;
    } else {
        return wide ? launch("moe_grouped_kernel<2,wide>", moe_grouped_kernel<BM, 2, true, kPartials, kFused, kI8, WT>, grid, kT, 0, s, gp)
                    : launch("moe_grouped_kernel<2>", moe_grouped_kernel<BM, 2, false, kPartials, kFused, kI8, WT>, grid, kT, 0, s, gp);
    }
}

// Q4_1 and Q8_0 weights: int8 block products, plain output or partials
template <int WT>
int launch_grouped_wt(int64_t bm, bool part, int vec, bool wide, const GroupedParams& gp, int64_t grid, hipStream_t s)
{
    switch (bm) {
    case 128: return part ? launch_grouped_v<128, true, false, true, WT>(vec, wide, gp, grid, s)
                          : launch_grouped_v<128, false, false, true, WT>(vec, wide, gp, grid, s);
    case 64: return part ? launch_grouped_v<64, true, false, true, WT>(vec, wide, gp, grid, s)
                         : launch_grouped_v<64, false, false, true, WT>(vec, wide, gp, grid, s);
    default: return part ? launch_grouped_v<32, true, false, true, WT>(vec, wide, gp, grid, s)
                         : launch_grouped_v<32, false, false, true, WT>(vec, wide, gp, grid, s);
    }
}

template <bool kPartials, bool kFused>
int launch_ws_v(int vec, bool wide, const GroupedParams& gp, int64_t grid, hipStream_t s)
{
    constexpr int kT = ws::kThreads;
    if (vec == 4) {
        return wide ? launch("moe_grouped_ws_kernel<4,wide>", ws::moe_grouped_ws_kernel<4, true, kPartials, kFused>, grid, kT, 0, s, gp)
                    : launch("moe_grouped_ws_kernel<4>", ws::moe_grouped_ws_kernel<4, false, kPartials, kFused>, grid, kT, 0, s, gp);
    }
    return wide ? launch("moe_grouped_ws_kernel<2,wide>", ws::moe_grouped_ws_kernel<2, true, kPartials, kFused>, grid, kT, 0, s, gp)
                : launch("moe_grouped_ws_kernel<2>", ws::moe_grouped_ws_kernel<2, false, kPartials, kFused>, grid, kT, 0, s, gp);
}

int launch_ws(bool part, bool fused, int vec, bool wide, const GroupedParams& gp, int64_t grid, hipStream_t s)
{
    if (part) return launch_ws_v<true, false>(vec, wide, gp, grid, s);
    if (fused) return launch_ws_v<false, true>(vec, wide, gp, grid, s);
    return launch_ws_v<false, false>(vec, wide, gp, grid, s);
}

template <int BM, bool kI8>
int launch_grouped(bool part, bool fused, int vec, bool wide, const GroupedParams& gp, int64_t grid, hipStream_t s)
{
    if (part) return launch_grouped_v<BM, true, false, kI8>(vec, wide, gp, grid, s);
    if (fused) return launch_grouped_v<BM, false, true, kI8>(vec, wide, gp, grid, s);
    return launch_grouped_v<BM, false, false, kI8>(vec, wide, gp, grid, s);
}

}  // namespace

int64_t grouped_tile_m(const MoeArgs& m)
{
    // FTQ_TILE_M=32|64|128 pins the tile height (tuning and tests); read once
    static const int64_t forced = [] {
        const char* v = getenv("FTQ_TILE_M");
        const int64_t t = v ? atoll(v) : 0;
        return (t == 32 || t == 64 || t == 128) ? t : 0;
    }();
    if (forced) return forced;
    // rows per M tile from the average pairs per expert (host arithmetic only)
    const int64_t per_expert = (m.T * m.top_k) / (m.E > 0 ? m.E : 1);
    if (per_expert >= 96) return 128;
    if (per_expert >= 40) return 64;
    return 32;
}

int run_grouped(const MoeArgs& m, const BucketPlan& plan, void* ws, hipStream_t s)
{
    if (plan.pairs == 0) return FTQ_OK;
    DeviceLimits lim;
    int st = device_limits(&lim);
    if (st != FTQ_OK) return st;
    uint8_t* base = static_cast<uint8_t*>(ws);
    const int64_t nb = m.K / kQK;
    const int64_t act_rows = m.T * m.top_k / m.act_div;   // tokens, or pairs
    GroupedParams gp{};
    gp.w = static_cast<const uint8_t*>(m.w);
    gp.a = static_cast<const uint8_t*>(m.a);
    gp.out = m.out;
    gp.partials = m.partials;
    gp.offsets = reinterpret_cast<const int32_t*>(base + plan.off_offsets);
    gp.tiles = reinterpret_cast<const int32_t*>(base + plan.off_tiles);
    gp.sorted = reinterpret_cast<const int32_t*>(base + plan.off_sorted);
    gp.tdesc = reinterpret_cast<const int4*>(base + plan.off_tdesc);
    gp.E = m.E;
    gp.N = m.N;
    gp.nb = nb;
    gp.top_k = m.top_k;
    gp.act_div = m.act_div;
    // buffer ranges: 32-bit unsigned byte counts (the narrow variant's activations are below 4 GiB)
    auto range32 = [](int64_t bytes) { return (int32_t)(uint32_t)std::min<int64_t>(bytes, UINT32_MAX); };
    gp.a_range = range32(act_rows * nb * kQ8Bytes);
    gp.act = m.act;
    gp.half = m.act ? m.N / 2 : 0;
    if (m.act) {
        // fused tiles address the gate and up rows from the expert's base
        if (m.N * nb * kQ4Bytes > (int64_t)UINT32_MAX) {
            set_error("fused activation on the grouped path: one expert's weights reach 4 GiB");
            return FTQ_ERR_UNSUPPORTED;
        }
        gp.wtile_range = range32(m.N * nb * kQ4Bytes);
        gp.n_tiles_n = (gp.half + kBN / 2 - 1) / (kBN / 2);
    } else {
        const int64_t wb = m.wtype == FTQ_W_Q8_0 ? w_bytes<FTQ_W_Q8_0>() : m.wtype == FTQ_W_Q4_1 ? w_bytes<FTQ_W_Q4_1>() : kQ4Bytes;
        if ((int64_t)kBN * nb * wb > (int64_t)UINT32_MAX) {
            set_error("grouped path: %d weight rows of K = %lld reach 4 GiB", kBN, (long long)m.K);
            return FTQ_ERR_UNSUPPORTED;
        }
        gp.wtile_range = range32((int64_t)kBN * nb * wb);
        gp.n_tiles_n = (m.N + kBN - 1) / kBN;
    }
    gp.nbuckets = plan.buckets;
    const int64_t bm = plan.tile_m;
    // sum over buckets of ceil(count/BM) <= (pairs + buckets*(BM-1)) / BM
    gp.max_mt = (plan.pairs + plan.buckets * (bm - 1)) / bm;
    const int64_t grid = std::min<int64_t>(gp.max_mt * gp.n_tiles_n, std::min<int64_t>(lim.max_grid_x, UINT32_MAX / kThreads));
    const uintptr_t wa = reinterpret_cast<uintptr_t>(m.w);
    // 4-byte weight loads where every pass's blocks start 4-byte aligned:
    // Q4_0 (18 B) and Q8_0 (34 B) pairs of blocks need K/32 even, Q4_1 (20 B)
    // blocks only aligned rows
    const int vec = (wa % 4 == 0 && (nb % 2 == 0 || m.wtype == FTQ_W_Q4_1)) ? 4 : 2;
    const bool part = m.partials != nullptr;
    // activation offsets fit 32 bits unless the staged activations reach 4 GiB;
    // FTQ_FORCE_WIDE=1 selects the 64-bit variant at any size (tests)
    static const bool force_wide = [] { const char* v = getenv("FTQ_FORCE_WIDE"); return v && v[0] == '1'; }();
    const bool wide = force_wide || act_rows * nb * kQ8Bytes >= ((int64_t)1 << 32);
    const bool fused = m.act != 0;
    // the block partials on int8 MFMAs by default; the fp16-MFMA kernels stay
    // selectable through ftq_debug_grouped_kernel for comparisons and tests
    if (m.wtype == FTQ_W_Q4_1) return launch_grouped_wt<FTQ_W_Q4_1>(bm, part, vec, wide, gp, grid, s);
    if (m.wtype == FTQ_W_Q8_0) return launch_grouped_wt<FTQ_W_Q8_0>(bm, part, vec, wide, gp, grid, s);
    const int variant = grouped_kernel_variant();
    const int64_t work_bound = gp.max_mt * gp.n_tiles_n;
    if (variant == kGroupedF16Ws && bm == 128 && work_bound < INT32_MAX) {
        int64_t g = std::min<int64_t>(work_bound, lim.cu_count);
        if (g >= kXcds) g -= g % kXcds;
        return launch_ws(part, fused, vec, wide, gp, std::max<int64_t>(g, 1), s);
    }
    if (variant == kGroupedI8) {
        switch (bm) {
        case 128: return launch_grouped<128, true>(part, fused, vec, wide, gp, grid, s);
        case 64: return launch_grouped<64, true>(part, fused, vec, wide, gp, grid, s);
        default: return launch_grouped<32, true>(part, fused, vec, wide, gp, grid, s);
        }
    }
    switch (bm) {
    case 128: return launch_grouped<128, false>(part, fused, vec, wide, gp, grid, s);
    case 64: return launch_grouped<64, false>(part, fused, vec, wide, gp, grid, s);
    default: return launch_grouped<32, false>(part, fused, vec, wide, gp, grid, s);
    }
}

}  // namespace ftq
