"""Shared helpers of the GPU tests: build one seeded case on both sides (each
side quantises the same fp32 tensors with its own code) and compare outputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from quantized_moe_expert_quantize_amd import ftq, inputs

U32 = 2.0 ** -24
U64 = 2.0 ** -53


def gamma(n, u):
    return n * u / (1 - n * u)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Case:
    """fp32 inputs from the shared generator; GPU and oracle quantise them independently."""

    def __init__(self, E, N, K, T, top_k, seed=0, kind="uniform", ids=None, x32=None, w32=None):
        self.E, self.N, self.K, self.T, self.top_k = E, N, K, T, top_k
        self.nb = K // 32
        self.w32 = inputs.weights(E, N, K, seed=seed) if w32 is None else w32
        self.x32 = inputs.activations(T, K, seed=seed) if x32 is None else x32
        self.ids = inputs.routing(T, E, top_k, seed=seed, kind=kind) if ids is None else np.ascontiguousarray(ids, np.int32)
        self._gpu = None
        self._orc = None

    # device side: libftq's own quantisers
    def gpu(self):
        if self._gpu is None:
            w = torch.from_numpy(self.w32).cuda()
            wq = ftq.quantize_q4_0(w)
            del w
            aq = ftq.quantize_q8_1(torch.from_numpy(self.x32).cuda())
            ids = torch.from_numpy(self.ids).cuda()
            self._gpu = (wq, aq, ids)
        return self._gpu

    # host side: the oracle's quantisers
    def orc(self):
        if self._orc is None:
            self._orc = (oracle.quantize_q4_0(self.w32).reshape(-1), oracle.quantize_q8_1(self.x32).reshape(-1))
        return self._orc

    def assert_same_bytes(self):
        wq, aq, _ = self.gpu()
        ow, oa = self.orc()
        assert np.array_equal(wq.cpu().numpy().reshape(-1), ow), "Q4_0 bytes differ from the oracle"
        assert np.array_equal(aq.cpu().numpy().reshape(-1), oa), "Q8_1 bytes differ from the oracle"

    def run(self, path=ftq.PATH_AUTO):
        wq, aq, ids = self.gpu()
        out = ftq.moe(wq, aq, ids, self.E, self.N, self.K, path=path)
        torch.cuda.synchronize()
        return out

    def partials(self, path):
        wq, aq, ids = self.gpu()
        p = ftq.moe_partials(wq, aq, ids, self.E, self.N, self.K, path=path)
        torch.cuda.synchronize()
        return p.cpu().numpy()

    def oracle_out(self, pairs=None):
        ow, oa = self.orc()
        if pairs is None:
            return oracle.moe(ow, oa, self.ids, self.E, self.N, self.K, self.T, self.top_k, want_abssum=True)
        return oracle.moe_pairs(ow, oa, self.ids, self.E, self.N, self.K, self.T, self.top_k, pairs, want_abssum=True)

    def oracle_partials(self):
        ow, oa = self.orc()
        return oracle.moe_partials(ow, oa, self.ids, self.E, self.N, self.K, self.T, self.top_k)


def assert_matches_oracle(gpu: np.ndarray, ref: np.ndarray, abssum: np.ndarray, nb: int):
    """Acceptance: rel-L2 <= 1e-5 and max-abs <= 1e-4 * max|ref|; and, per element,
    the rigorous fp32 summation bound |gpu - exact| <= gamma_{nb+2}(2^-24) * sum|terms|
    (any summation order, one rounding per block term), widened by the oracle's
    own fp64 error."""
    gpu = gpu.astype(np.float64)
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu))
    diff = np.abs(gpu - ref)
    bound = (gamma(nb + 2, U32) + gamma(nb, U64)) * abssum
    worst = np.argmax(diff - bound)
    assert np.all(diff <= bound), f"element {np.unravel_index(worst, diff.shape)}: |diff|={diff.flat[worst]:.3e} > bound {bound.flat[worst]:.3e}"
    nref = np.linalg.norm(ref)
    if nref > 0:
        rel = np.linalg.norm(gpu - ref) / nref
        assert rel <= 1e-5, f"relative L2 error {rel:.3e}"
        assert diff.max() <= 1e-4 * np.abs(ref).max()
    else:
        assert diff.max() == 0


def sample_pairs(T, top_k, n, seed=0):
    pairs = T * top_k
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(pairs, size=min(n, pairs), replace=False).tolist())
    pick.update({0, pairs - 1})
    return np.array(sorted(pick), np.int64)
