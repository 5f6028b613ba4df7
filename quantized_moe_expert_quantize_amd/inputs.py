"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module draws random numbers only: fp32 weights, fp32 activations and
top-k routing ids and gate weights.  It holds none of the method's arithmetic (no quantisation,
no dot products); each side quantises the fp32 tensors with its own code.

Recipe (the pages run real checkpoints that are not available, so seeded
synthetic tensors with the same shapes stand in for them):
  * one numpy PCG64 stream per tensor: SeedSequence([seed, tensor_id]) with
    tensor ids weights=0, activations=1, routing=2, gates=3;
  * weights   fp32 N(0, 0.02), shape [E, N, K];
  * activations fp32 N(0, 1), shape [T, K];
  * routing: per token, top_k DISTINCT experts.  "uniform": every k-subset
    equally likely (argsort of iid uniforms); "zipf": expert r drawn with
    weight (r+1)^-s, k distinct by successive weighted sampling without
    replacement (Gumbel-top-k);
  * gates fp32 [T, top_k]: iid U(0.05, 1) per slot, scaled so each token's
    row sums to about one (routing weights after a top-k softmax);
  * gguf_blocks: uniformly random code bytes with fp16 scales ~ U(1e-3, 2e-3)
    (and offsets ~ U(-0.03, -0.01)) in the GGUF block layouts, for timing
    the other weight types without a quantizer (tensor id 4).
Shapes of the pages' workloads: FreeToken PR #185 "Performance" (nrows=1408,
hidden=2816, top_k=8, 128 experts) and mlxcel PR #652 "Summary"
(qwen3-30b-a3b at 8192 tokens, mixtral-8x7b at 32768 tokens).
"""
from __future__ import annotations

import numpy as np

WEIGHTS, ACTIVATIONS, ROUTING, GATES, BLOCKS = 0, 1, 2, 3, 4


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id)]))


def weights(E: int, N: int, K: int, seed: int = 0, std: float = 0.02) -> np.ndarray:
    """fp32 [E, N, K] ~ N(0, std^2)."""
    g = _rng(seed, WEIGHTS)
    w = g.standard_normal((E, N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def activations(T: int, K: int, seed: int = 0) -> np.ndarray:
    """fp32 [T, K] ~ N(0, 1)."""
    return _rng(seed, ACTIVATIONS).standard_normal((T, K), dtype=np.float32)


def routing(T: int, E: int, top_k: int, seed: int = 0, kind: str = "uniform",
            zipf_s: float = 1.1) -> np.ndarray:
    """int32 [T, top_k] expert ids, distinct within each token."""
    if top_k > E:
        raise ValueError("top_k must not exceed the number of experts")
    g = _rng(seed, ROUTING)
    if T == 0:
        return np.zeros((0, top_k), np.int32)
    if kind == "uniform":
        u = g.random((T, E))
        ids = np.argsort(u, axis=1, kind="stable")[:, :top_k]
    elif kind == "zipf":
        logw = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        gumbel = -np.log(-np.log(g.random((T, E))))
        ids = np.argsort(-(logw[None, :] + gumbel), axis=1, kind="stable")[:, :top_k]
    else:
        raise ValueError(f"unknown routing kind {kind!r}")
    return np.ascontiguousarray(ids, dtype=np.int32)


def gguf_blocks(wtype: int, E: int, N: int, K: int, seed: int = 0) -> np.ndarray:
    """uint8 [E, N, K/32 * block bytes] of random valid blocks of GGUF type
    wtype (3 Q4_1, 6 Q5_0, 7 Q5_1, 8 Q8_0; scale fp16 at byte 0, offset fp16 at
    byte 2 for Q4_1/Q5_1); every other byte uniformly random."""
    size = {2: 18, 3: 20, 6: 22, 7: 24, 8: 34}[wtype]
    g = _rng(seed, BLOCKS)
    nblk = E * N * (K // 32)
    b = g.integers(0, 256, (nblk, size), dtype=np.uint8)
    b[:, 0:2] = g.uniform(1e-3, 2e-3, nblk).astype(np.float16).view(np.uint8).reshape(nblk, 2)
    if wtype in (3, 7):
        b[:, 2:4] = g.uniform(-0.03, -0.01, nblk).astype(np.float16).view(np.uint8).reshape(nblk, 2)
    return b.reshape(E, N, K // 32 * size)


def gates(T: int, top_k: int, seed: int = 0) -> np.ndarray:
    """fp32 [T, top_k] positive weights, each row summing to about one."""
    g = _rng(seed, GATES).uniform(0.05, 1.0, (T, top_k))
    return np.ascontiguousarray(g / g.sum(axis=1, keepdims=True), dtype=np.float32)


# The workloads, by name.  Each entry: E, top_k, K (hidden), N (rows per
# expert), token counts, routing kind.
WORKLOADS = {
    "tiny": dict(E=8, top_k=2, K=256, N=128, T=(16,), routing="uniform"),
    "page1": dict(E=128, top_k=8, K=2816, N=1408, T=(2048, 4096, 8191), routing="uniform"),
    "page1_overcap": dict(E=128, top_k=8, K=2816, N=1408, T=(8192, 16384), routing="uniform"),
    "qwen3_30b_a3b_up": dict(E=128, top_k=8, K=2048, N=768, T=(8192,), routing="zipf"),
    "mixtral_8x7b": dict(E=8, top_k=2, K=4096, N=14336, T=(1, 8, 64, 32768), routing="uniform"),
}
