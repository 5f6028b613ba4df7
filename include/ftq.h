/*
 * ftq.h -- C ABI of libftq: the mixture-of-experts expert matmul with 4-bit
 * block-quantized weights (Q4_0) against 8-bit block-quantized activations
 * (Q8_1) on AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  For every flat (token, top-k) pair
 * p = t*top_k + j, with e = topk_ids[t][j]:
 *
 *     out[p][n] = sum over blocks b of  P[p][n][b] * d4[e][n][b] * d8[t][b]
 *     P[p][n][b] = sum_{i<32} (q4[e][n][b][i] - 8) * q8[t][b][i]     (exact int)
 *
 * i.e. the routed expert's Q4_0 rows dotted with the token's Q8_1 row, one
 * output row per pair.  This is the MoE GEMV of FreeToken PR #185 ("fix(kernel):
 * launch GGUF MoE GEMV token axis on grid.x, not grid.z", sections Problem and
 * Fix), generalised so that batches of any size run, with no 65535-pair limit
 * and 64-bit size arithmetic (mlxcel PR #652, "fix(cuda/quantized): chunk
 * long-prompt qmm launches to avoid gridDim>65535 and int overflow", Summary).
 *
 * Block formats (GGUF; the pages name them, the layouts are the GGUF ones):
 *   Q4_0 block, 18 bytes: fp16 d, then 16 bytes; byte i holds element i in its
 *       low nibble and element i+16 in its high nibble; value = (nibble-8)*d.
 *   Q8_1 block, 36 bytes: fp16 d, fp16 s, then 32 int8 q; value = q*d and
 *       s = d * sum(q).  The matmul reads d and q only.
 *
 * Conventions shared by every entry point:
 *   - Sizes are int64_t.  Pointers are device pointers on the current HIP
 *     device unless stated.  Work is enqueued on `stream` (0 = null stream);
 *     no call synchronises, allocates, frees or reads device data back to the
 *     host, so every call may be recorded into a HIP graph.
 *   - The caller owns every buffer.  The library writes only the outputs and
 *     the workspace named in each call.
 *   - Arguments are validated before anything is enqueued; on a bad argument
 *     nothing is launched and FTQ_ERR_INVALID_ARG (or FTQ_ERR_UNSUPPORTED /
 *     FTQ_ERR_WORKSPACE) is returned.
 *   - Every kernel launch is checked immediately after it is issued; a
 *     rejected launch returns FTQ_ERR_LAUNCH and ftq_last_error() names the
 *     kernel, grid, block and LDS bytes (FreeToken PR #185, Fix: a rejected
 *     launch reports the geometry that caused it instead of latching).  The
 *     error is cleared, so the next call is unaffected.  Faults during
 *     execution surface at the caller's next synchronisation, as for any
 *     asynchronous HIP work.
 *   - No C++ exception crosses this interface.
 */
#ifndef FTQ_H
#define FTQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FTQ_OK = 0,
    FTQ_ERR_INVALID_ARG = 1,  /* bad size, null or misaligned pointer        */
    FTQ_ERR_WORKSPACE = 2,    /* workspace missing or smaller than required  */
    FTQ_ERR_LAUNCH = 3,       /* a kernel launch was rejected               */
    FTQ_ERR_UNSUPPORTED = 4,  /* valid request this build does not handle    */
    FTQ_ERR_HIP = 5           /* a HIP runtime query failed                  */
} ftq_status;

typedef enum {
    FTQ_PATH_AUTO = 0,        /* chosen on the host from the sizes alone     */
    FTQ_PATH_GEMV = 1,        /* memory-bound path for few pairs per expert  */
    FTQ_PATH_GROUPED = 2      /* expert-sorted MFMA tiles for prefill        */
} ftq_path;

/* Weight block types, with the type ids GGUF files use (see ftq_moe_gguf_q8_1). */
typedef enum {
    FTQ_W_Q4_0 = 2,           /* 18 B: fp16 d, 16 nibble bytes           w = (q - 8) d  */
    FTQ_W_Q4_1 = 3,           /* 20 B: fp16 d, fp16 m, 16 nibble bytes   w = q d + m    */
    FTQ_W_Q5_0 = 6,           /* 22 B: fp16 d, 32-bit qh, nibble bytes   w = (q - 16) d */
    FTQ_W_Q5_1 = 7,           /* 24 B: fp16 d, fp16 m, qh, nibble bytes  w = q d + m    */
    FTQ_W_Q8_0 = 8            /* 34 B: fp16 d, 32 int8                   w = q d        */
} ftq_wtype;

typedef enum {
    FTQ_ACT_SILU = 1,         /* x / (1 + exp(-x))                           */
    FTQ_ACT_GELU_TANH = 2     /* x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
} ftq_act;

#define FTQ_QK 32
#define FTQ_Q4_0_BLOCK_BYTES 18
#define FTQ_Q8_1_BLOCK_BYTES 36

/*
 * Quantize fp32 activations to Q8_1 (the activation quantiser that runs before
 * the MoE GEMV; FreeToken PR #185, Fix, "quantize_row_q8_1_cuda").
 *   x: fp32 [T][K], row-major, 16-byte aligned.      K % 32 == 0, T >= 0.
 *   y: [T][K/32] Q8_1 blocks (36 B each), 4-byte aligned, written.
 * Per 32-value block: amax = max|x|, d = amax/127 (fp32, IEEE division),
 * q = round-half-away-from-zero(x/d) (0 when amax == 0), s = d*sum(q) in fp32;
 * d and s stored as fp16 (round to nearest even).  Bit-exact and deterministic.
 * T == 0 is a no-op.  Any number of rows: the launch has no 65535 limit.
 */
int ftq_quantize_q8_1(const float* x, int64_t T, int64_t K, void* y, hipStream_t stream);

/*
 * Quantize fp32 weights to Q4_0 (weight preparation; not part of the matmul).
 *   w: fp32 [rows][K], 16-byte aligned.  K % 32 == 0.
 *   y: [rows][K/32] Q4_0 blocks (18 B each), 2-byte aligned, written.
 * Per block: m = the element of largest magnitude (first on ties), d = m/-8,
 * q = clamp(round-half-away(x/d) + 8, 0, 15) (8 when d == 0); d stored fp16.
 */
int ftq_quantize_q4_0(const float* w, int64_t rows, int64_t K, void* y, hipStream_t stream);

/*
 * The path FTQ_PATH_AUTO takes for these sizes (FTQ_PATH_GEMV or
 * FTQ_PATH_GROUPED), or -FTQ_ERR_INVALID_ARG for invalid sizes.  Pure host
 * arithmetic on E, T and top_k: the choice never reads device data, so no
 * call has to wait for the GPU and every call stays capturable in a graph
 * ("Current Bug: CuTeDSLMoERunner", Bug 8b and Cudagraph Constraints: a host
 * readback of device values breaks capture).  Rule: the GEMV path when
 * T*top_k <= 4096 and the pairs per expert T*top_k/E are at most 7 (E <= 16)
 * or 4 (E > 16); the grouped path otherwise.
 * Bit equality of a batch and its split halves (FreeToken PR #185, Test) holds
 * on each forced path.  Under FTQ_PATH_AUTO it holds when the batch and its
 * halves fall on the same side of the rule, which is not the case just above
 * the crossover: with 128 experts and top_k = 8, T = 65..128 runs grouped and
 * its halves run the GEMV; with 8 experts and top_k = 2, T = 29..56.  The two
 * paths sum in different orders, so their bits differ there (both within the
 * stated tolerance of the exact result).
 */
int ftq_moe_select_path(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k);

/*
 * Exact workspace size in bytes that ftq_moe_q4_0_q8_1 needs for these sizes
 * and this path (FTQ_PATH_AUTO resolved as above); 0 means none.  Returns -1
 * for invalid sizes (ftq_last_error says why).  Host arithmetic only, from the
 * same sizes the call takes, so the caller can allocate it once per shape.
 * The bound is exact rather than a guess at a maximum because buffers sized
 * from the wrong bound are what broke the expert-sorted runner of "Current
 * Bug: CuTeDSLMoERunner" (Bug 9: a padded buffer too small, indexed out of
 * bounds; Bug 15: buffers sized for the largest batch, out of memory; Bug 16:
 * a buffer sized for max_tokens*top_k where the layout needed
 * num_experts*max_chunks*128).  What it holds: per-chunk bucket counts, the
 * per-expert segment and tile offsets and the sorted pair list, each 256-byte
 * aligned; it grows with T*top_k and E, not with N or K.
 */
int64_t ftq_moe_workspace_bytes(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path);

/*
 * The MoE expert matmul.
 *   w:        [E][N][K/32] Q4_0 blocks (expert e, row n, block b at byte
 *             ((e*N + n)*(K/32) + b)*18), 2-byte aligned.
 *   a:        [T][K/32] Q8_1 blocks, 4-byte aligned (ftq_quantize_q8_1 output).
 *   topk_ids: int32 [T][top_k], 4-byte aligned.  Ids outside [0, E) give an
 *             all-zero output row (masking of non-local experts, "Current Bug:
 *             CuTeDSLMoERunner", Bug 8).  Repeated ids are allowed.
 *   out:      fp32 [T*top_k][N], row p = t*top_k + j, 4-byte aligned, written.
 *   workspace: device scratch of at least ftq_moe_workspace_bytes(...) bytes,
 *             256-byte aligned (may be NULL when that is 0).  Its contents on
 *             entry do not matter; calls sharing one workspace must not overlap.
 *   path:     FTQ_PATH_AUTO, FTQ_PATH_GEMV or FTQ_PATH_GROUPED.  Both paths
 *             compute the same exact block products and sum them in fp32,
 *             in different orders.  Each forced path is deterministic and
 *             batch invariant: a row's bits depend neither on the other rows
 *             nor on the batch size.  Which path FTQ_PATH_AUTO takes does
 *             depend on the batch size (ftq_moe_select_path).
 * Limits: K % 32 == 0; E, N, top_k >= 1; top_k <= E; E <= 4095 (the bucket
 * tables live in LDS: FTQ_ERR_UNSUPPORTED above); T >= 0 (T == 0: no-op);
 * T*top_k < 2^31.  Output offsets use 64-bit arithmetic throughout.
 */
int ftq_moe_q4_0_q8_1(const void* w, const void* a, const int32_t* topk_ids, float* out,
                      int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                      void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

/*
 * ftq_moe_q4_0_q8_1 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace argument: the workspace that ftq_moe_q4_0_q8_1 would need
 * lives in a fixed 4 MiB array that the library holds on each device it runs
 * on, until the process ends.  Arguments, results, path choice and errors are
 * those of ftq_moe_q4_0_q8_1 (the results are bit-identical to it), and:
 *   - FTQ_ERR_UNSUPPORTED when ftq_moe_workspace_bytes(E, N, K, T, top_k, path)
 *     exceeds 4 MiB (e.g. above about 900 000 pairs with 128 experts);
 *   - FTQ_ERR_HIP if the array's device address cannot be obtained (looked up
 *     once per device, on the first call with that device current).
 * Nothing is allocated or freed and nothing needs clearing between calls.  All
 * calls on one device share the array: calls that may overlap on one device
 * (several streams or host threads) race on it and must be serialised by the
 * caller.
 */
int ftq_moe_q4_0_q8_1_noalloc(const void* w, const void* a, const int32_t* topk_ids, float* out,
                              int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path,
                              hipStream_t stream);

/*
 * The same matmul split in two, so that one routing can serve several matmuls
 * over the same (token, top-k) pairs (e.g. an expert FFN's up- and
 * down-projections) and each half can be timed on its own.
 *
 * ftq_moe_route: groups the pairs by routed expert into `workspace` (per-expert
 *   counts, segment offsets, tile table and the sorted pair list: the
 *   expert-sorted layout of "Current Bug: CuTeDSLMoERunner", Key Architecture,
 *   built on the device without any host readback).  Pass the workspace and
 *   path that the matmul will use (ftq_moe_workspace_bytes with the matmul's
 *   N and K; the routing itself uses only its leading part, which depends on
 *   E, T and top_k alone).  A path that needs no workspace makes this a no-op.
 * ftq_moe_q4_0_q8_1_routed: the matmul on pairs routed by ftq_moe_route with
 *   the same topk_ids, E, T, top_k, path and workspace, enqueued after it.
 *   Arguments and results are exactly those of ftq_moe_q4_0_q8_1.
 */
int ftq_moe_route(const int32_t* topk_ids, int64_t E, int64_t T, int64_t top_k, void* workspace,
                  size_t workspace_bytes, int path, hipStream_t stream);

int ftq_moe_q4_0_q8_1_routed(const void* w, const void* a, const int32_t* topk_ids, float* out,
                             int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                             void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

/*
 * Checking aid: the same computation, but instead of the fp32 outputs it
 * writes the exact integer block partials
 *   partials: int32 [T*top_k][N][K/32], P[p][n][b] as defined above
 * (zeros for masked pairs), produced by the chosen path's own kernels and
 * index arithmetic.  Same arguments, limits and workspace as above.
 */
int ftq_moe_q4_0_q8_1_partials(const void* w, const void* a, const int32_t* topk_ids,
                               int32_t* partials, int64_t E, int64_t N, int64_t K, int64_t T,
                               int64_t top_k, void* workspace, size_t workspace_bytes, int path,
                               hipStream_t stream);

/*
 * Per-pair activations: the down projection of an expert FFN.  ("Current Bug:
 * CuTeDSLMoERunner", Bug 6: the second layer consumes what the first produced
 * for each routed pair, so its input is one row per pair, not per token.)
 *
 * Same as ftq_moe_q4_0_q8_1 / _routed / _partials except for the activations:
 *   a_pairs  Q8_1 blocks [T*top_k][K/32] (row p = t*top_k + j feeds pair p
 *            only; 4-byte aligned).
 * Outputs, routing, limits, errors and determinism are as documented above;
 * a masked pair's row is zero whatever its activation row holds.  The grouped
 * path stages one row per pair, so these calls need
 * ftq_moe_pairs_workspace_bytes(...) bytes of workspace (the same as
 * ftq_moe_workspace_bytes for the GEMV path).  A routing made by ftq_moe_route
 * serves these calls too, when the workspace has this size.
 */
int64_t ftq_moe_pairs_workspace_bytes(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int path);

int ftq_moe_q4_0_q8_1_pairs(const void* w, const void* a_pairs, const int32_t* topk_ids, float* out,
                            int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                            void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

int ftq_moe_q4_0_q8_1_pairs_routed(const void* w, const void* a_pairs, const int32_t* topk_ids,
                                   float* out, int64_t E, int64_t N, int64_t K, int64_t T,
                                   int64_t top_k, void* workspace, size_t workspace_bytes, int path,
                                   hipStream_t stream);

int ftq_moe_q4_0_q8_1_pairs_partials(const void* w, const void* a_pairs, const int32_t* topk_ids,
                                     int32_t* partials, int64_t E, int64_t N, int64_t K, int64_t T,
                                     int64_t top_k, void* workspace, size_t workspace_bytes, int path,
                                     hipStream_t stream);

/*
 * Top-k weighted combine: the expert FFN's output per token.
 *
 *   out[t][n] = sum_{j < top_k} gates[t][j] * y[t*top_k + j][n]
 *
 *   y      fp32 [T*top_k][N], row p = t*top_k + j (the layout every matmul entry
 *          point writes; masked pairs' rows are zero and add nothing)
 *   gates  fp32 [T][top_k], the router's weights, any values
 *   out    fp32 [T][N]; must not overlap y or gates
 * Evaluated in fp32 as acc = fma(gates[t][j], y[t*top_k+j][n], acc) for
 * j = 0 .. top_k-1 from acc = +0: a fixed order, so the result is bit-exact
 * across calls and independent of how the batch is split; with top_k = 1 and
 * gates = 1 it reproduces y exactly.
 * All pointers 4-byte aligned device pointers (16-byte alignment and N % 4 == 0
 * select 16-byte accesses).  T = 0 is a no-op.  Errors: FTQ_ERR_INVALID_ARG
 * (T < 0, top_k < 1, N < 1, null or misaligned pointers), FTQ_ERR_UNSUPPORTED
 * (T*top_k*N*8 overflows int64), FTQ_ERR_LAUNCH.
 */
int ftq_moe_combine_topk(const float* y, const float* gates, float* out, int64_t T, int64_t top_k,
                         int64_t N, hipStream_t stream);

/*
 * The first layer of an expert FFN with its gated activation fused into the
 * matmul's epilogue: the GEMV's output feeds gelu_tanh_and_mul in FreeToken
 * PR #185 (Problem), and the second layer's input is the output "after
 * SiLU*up" in "Current Bug: CuTeDSLMoERunner" (Bug 6).  Each expert's N weight
 * rows are [gate rows 0..N/2-1 | up rows N/2..N-1] (the order of the halves is
 * this library's reading; the pages print no layout).  For pair p and output
 * column c < N/2:
 *
 *   out[p][c] = act(y[p][c]) * y[p][N/2 + c],  y[p][n] the plain matmul value
 *
 * computed in fp32 from the matmul's fp32 gate and up values, without writing
 * y.  Both activations are evaluated as x * 1/(1 + e^-z), with z = x for SiLU
 * and z = 2 sqrt(2/pi) (x + 0.044715 x^3) for the tanh form of GELU (the same
 * function, since (1 + tanh(z/2))/2 = 1/(1 + e^-z)); e^-z is one hardware
 * base-2 exponential and the quotient one hardware reciprocal.  Relative to the
 * exact activation of the fp32 inputs the result is within 9 u (|act(x)| + |x|),
 * u = 2^-24, which the tests check together with the matmul's own bound.  Arguments are those of ftq_moe_q4_0_q8_1 (per-token
 * activations, the same workspace: ftq_moe_workspace_bytes(E, N, K, ...)), plus
 *   N:    weight rows per expert, even (gate and up halves);
 *   act:  FTQ_ACT_SILU or FTQ_ACT_GELU_TANH;
 *   out:  fp32 [T*top_k][N/2], row p = t*top_k + j; masked pairs give zero rows.
 * Errors: N odd or act unknown: FTQ_ERR_INVALID_ARG.  FTQ_ERR_UNSUPPORTED when
 * one expert's weights reach 4 GiB (grouped path) or when one activation row
 * does not fit the GEMV path's on-chip staging (K beyond 33 056 with 8 experts,
 * 32 000 with 128; the per-expert tables share the budget).
 * ftq_moe_q4_0_q8_1_act_routed takes pairs routed by ftq_moe_route, as
 * ftq_moe_q4_0_q8_1_routed does.
 */
int ftq_moe_q4_0_q8_1_act(const void* w, const void* a, const int32_t* topk_ids, float* out,
                          int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int act,
                          void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

int ftq_moe_q4_0_q8_1_act_routed(const void* w, const void* a, const int32_t* topk_ids, float* out,
                                 int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int act,
                                 void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

/*
 * The matmul for the other GGUF weight block types that FreeToken PR #185
 * (Problem) counts among the GEMV's sibling launchers: Q4_1, Q5_0, Q5_1 and
 * Q8_0 (layouts in ftq_wtype; the pages name the types but print no layout:
 * these are the GGUF layouts), against Q8_1 activations.  For pair p, row n:
 *
 *   out[p][n] = sum_b ( d[n][b] * d8[b] * sum_i (q[n][b][i] - z) * q8[b][i]
 *                     + m[n][b] * d8[b] * sum_i q8[b][i] )
 *
 * z the zero point (8 for Q4_0, 16 for Q5_0, else 0) and m the offset (Q4_1,
 * Q5_1; else 0): the dot product of the dequantised weights and activations.
 * The integer sums are exact; the offset term uses the exact integer sum of
 * the activation codes, not the fp16 s field.  Evaluation in fp32.  GEMV path:
 * per block acc = fma(P, d*d8, acc) then, for offset types, acc = fma(S,
 * m*d8, acc), S = sum q8.  Grouped path: per block acc = fma(P, d*d8, acc) with
 * P from an int8 matrix product; the Q4_1 offset terms of each pass of two
 * blocks are added into acc by one bf16 matrix product whose operands split
 * d8*S (exact in fp32) and m into bf16 pieces with exact products (only the
 * sums round).
 *   w:          [E][N][K/32] blocks of wtype;
 *   a:          Q8_1, [T][K/32] (act_per_pair == 0) or [T*top_k][K/32] (one
 *               row per pair, as ftq_moe_q4_0_q8_1_pairs);
 *   other arguments as ftq_moe_q4_0_q8_1; the workspace is
 *   ftq_moe_workspace_bytes(E, N, K, T, top_k, path) bytes.
 * FTQ_W_Q4_0 runs the Q4_0 paths.  Q4_1 and Q8_0 run on both paths, chosen as
 * for Q4_0 under FTQ_PATH_AUTO (the grouped path at prefill sizes); Q5_0 and
 * Q5_1 on the GEMV path only (FTQ_PATH_AUTO selects it; FTQ_PATH_GROUPED returns
 * FTQ_ERR_UNSUPPORTED).  Weight rows that are not 4-byte aligned (Q5_0 and
 * Q8_0 with an odd K/32) return FTQ_ERR_UNSUPPORTED on either path.  Unknown
 * wtype: FTQ_ERR_INVALID_ARG.
 * ftq_moe_gguf_q8_1_partials writes the integer parts sum((q - z) * q8) as
 * int32 [T*top_k][N][K/32] instead (checking aid).
 */
int ftq_moe_gguf_q8_1(const void* w, int wtype, const void* a, const int32_t* topk_ids, float* out,
                      int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int act_per_pair,
                      void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

int ftq_moe_gguf_q8_1_partials(const void* w, int wtype, const void* a, const int32_t* topk_ids,
                               int32_t* partials, int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k,
                               int act_per_pair, void* workspace, size_t workspace_bytes, int path,
                               hipStream_t stream);

/*
 * Message for the last failing call on this thread ("" if none): for a
 * rejected launch it names the kernel, grid, block and LDS bytes and the HIP
 * error (FreeToken PR #185, Fix: report the geometry of a failed launch).  The
 * pointer stays valid until the next ftq_* call on the same thread; every call
 * clears it on entry.
 */
const char* ftq_last_error(void);

/* Library version string, e.g. "ftq 0.1.0 gfx950". */
const char* ftq_version(void);

/*
 * Test hook: while `threads` > 0, every launch on this thread asks for
 * `threads` threads per block, so that a geometry the device rejects can be
 * exercised from the host.  The library's own pre-launch geometry check turns
 * it into FTQ_ERR_LAUNCH before anything is enqueued.  0 restores normal
 * operation.
 */
void ftq_debug_force_block_threads(int threads);

/*
 * Comparison hook: which kernel the grouped path launches for later calls on
 * this host thread.  0 (the default): exact block partials on int8 MFMAs
 * (v_mfma_i32_32x32x32_i8 on the nibble codes minus 8 and the Q8_1 codes),
 * converted to fp32 before the scale FMA.  1: the same partials as two fp16
 * MFMAs (the codes are exact in fp16).  2: the fp16 partials in a
 * warp-specialised kernel (loader and MMA waves paced by LDS counters instead
 * of workgroup barriers; 128-row tiles only, else as 1).  All three produce
 * the same integer partials and the same fp32 outputs bit for bit; they differ
 * in speed only.  Returns FTQ_OK, or FTQ_ERR_INVALID_ARG for another value.
 */
int ftq_debug_grouped_kernel(int variant);

/*
 * Comparison hook: with `split` non-zero, later routings on this host thread
 * (ftq_moe_route and the routing inside the matmul calls) always run the
 * bucketing as three kernels (per-chunk counts, one scan, the in-order
 * scatter); with 0 (the default), batches of at most 8192 pairs whose
 * per-chunk counts fit on chip (buckets x chunks <= 8192, at most 2048
 * buckets) run the same three passes in one workgroup instead.  Both build
 * the same tables bit for bit; they differ in speed only.
 */
void ftq_debug_route_kernels(int split);

/*
 * Checking aid: the on-chip plan the GEMV path makes for these sizes, host
 * arithmetic only (no device is touched).  *seg: K/32 blocks staged per
 * segment (less than K/32 when a row is streamed in several K segments, which
 * happens when the activation rows of the pairs served per pass do not fit in
 * LDS next to the weight buffers); *pairs_per_pass: activation rows staged per
 * pass; *wg_per_cu: workgroups per CU.  wtype as ftq_wtype, act 0 or FTQ_ACT_*.
 * Returns FTQ_OK, or the error the matmul would return for these sizes.
 */
int ftq_debug_gemv_plan(int64_t E, int64_t N, int64_t K, int64_t T, int64_t top_k, int wtype, int act,
                        int64_t* seg, int64_t* pairs_per_pass, int64_t* wg_per_cu);

#ifdef __cplusplus
}
#endif

#endif /* FTQ_H */
