"""The GEMV path on rows longer than its on-chip staging: K segments.

When the activation rows of the pairs served in one pass do not fit in LDS
next to the weight buffers, the GEMV streams each weight row in several K
segments, continuing each row's running sum through the output.  AUTO reaches
this on the Mixtral down projection (mlxcel PR #652, Summary: mixtral-8x7b;
the second layer's K is the expert width 14336 and its input one row per pair,
"Current Bug: CuTeDSLMoERunner", Bug 6) at T = 12 and 16, where each expert
holds 3-4 pairs.  Every shape here is first checked to plan several segments
(host arithmetic of the library itself), so the tests cannot drift back to one.

Bar: integer block partials bit-exact; fp32 outputs within the stated
tolerance of the oracle; a batch and its split halves bit-equal on the GEMV
path (FreeToken PR #185, Test), although the halves stage whole rows in one
segment and the batch does not."""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_quantize_amd import ftq, inputs
from tests._cases import Case, assert_matches_oracle, say
from tests.test_gpu_down import PairCase

pytestmark = pytest.mark.gpu

MIXTRAL_DOWN = (8, 4096, 14336, 2)   # E, N (hidden), K (expert width), top_k


def _assert_segmented(E, N, K, T, k, wtype=2):
    plan = ftq.gemv_plan(E, N, K, T, k, wtype)
    say(f"[kseg] E={E} N={N} K={K} T={T} top_k={k} wtype={wtype}: plan {plan}")
    assert plan["seg"] < K // 32, plan
    return plan


@pytest.mark.parametrize("T", [12, 16])
@pytest.mark.parametrize("path", [ftq.PATH_AUTO, ftq.PATH_GEMV])
def test_mixtral_down_segmented_rows_match_oracle(T, path):
    E, N, K, k = MIXTRAL_DOWN
    _assert_segmented(E, N, K, T, k)
    assert ftq.select_path(E, N, K, T, k) == ftq.PATH_GEMV
    c = PairCase(E, N, K, T, k, seed=4)
    got = c.run(path).cpu().numpy()
    pairs = np.arange(T * k)   # every pair: the oracle computes these one by one in seconds
    ref, ab = c.oracle_out(pairs)
    assert_matches_oracle(got[pairs], ref, ab, c.nb)


def test_mixtral_down_segmented_partials_bit_exact():
    # the same K and routing with fewer rows: the plan depends on E, K, T and
    # top_k only, so the rows are still streamed in segments
    E, N, K, k = MIXTRAL_DOWN
    N, T = 96, 16
    _assert_segmented(E, N, K, T, k)
    c = PairCase(E, N, K, T, k, seed=4)
    assert np.array_equal(c.partials(ftq.PATH_GEMV), c.oracle_partials())


def test_mixtral_down_segmented_batch_equals_its_halves():
    E, N, K, k = MIXTRAL_DOWN
    T = 16
    _assert_segmented(E, N, K, T, k)
    assert ftq.gemv_plan(E, N, K, T // 2, k)["seg"] == K // 32   # the halves: one segment
    c = PairCase(E, N, K, T, k, seed=6)
    wq, aq, ids = c.gpu()
    for path in (ftq.PATH_GEMV, ftq.PATH_AUTO):
        whole = ftq.moe_pairs(wq, aq, ids, E, N, K, path=path)
        h = T // 2
        lo = ftq.moe_pairs(wq, aq[: h * k].contiguous(), ids[:h].contiguous(), E, N, K, path=path)
        hi = ftq.moe_pairs(wq, aq[h * k:].contiguous(), ids[h:].contiguous(), E, N, K, path=path)
        torch.cuda.synchronize()
        assert torch.equal(whole, torch.cat([lo, hi])), f"path {path}"


def test_long_rows_per_token_activations():
    # per-token activations, K = 20480 (640 blocks: segments of 256, 256, 128)
    # with 4 pairs per expert, on the GEMV path forced
    E, N, K, T, k = 4, 48, 20480, 8, 2
    _assert_segmented(E, N, K, T, k)
    c = Case(E, N, K, T, k, seed=8)
    c.assert_same_bytes()
    assert np.array_equal(c.partials(ftq.PATH_GEMV), c.oracle_partials())
    ref, ab = c.oracle_out()
    assert_matches_oracle(c.run(ftq.PATH_GEMV).cpu().numpy(), ref, ab, c.nb)


def test_long_rows_q8_0_weights():
    # a sibling block type through the same segmented stream
    E, N, K, T, k = 4, 40, 20480, 8, 2
    wt = ftq.W_Q8_0
    _assert_segmented(E, N, K, T, k, wt)
    wb = oracle.quantize_w(wt, inputs.weights(E, N, K, seed=2) * np.float32(40.0)).reshape(-1)
    x32 = inputs.activations(T, K, seed=9)
    ids = inputs.routing(T, E, k, seed=2)
    oa = oracle.quantize_q8_1(x32).reshape(-1)
    w_d, ids_d = torch.from_numpy(wb).cuda(), torch.from_numpy(ids).cuda()
    a_d = ftq.quantize_q8_1(torch.from_numpy(x32).cuda())
    assert np.array_equal(a_d.cpu().numpy().reshape(-1), oa)
    part = ftq.moe_gguf_partials(w_d, wt, a_d, ids_d, E, N, K).cpu().numpy()
    ref_part = oracle.moe_w_partials(wt, wb, oa, ids, E, N, K, T, k)
    assert np.array_equal(part, ref_part)
    got = ftq.moe_gguf(w_d, wt, a_d, ids_d, E, N, K, path=ftq.PATH_GEMV).cpu().numpy()
    ref, ab = oracle.moe_w(wt, wb, oa, ids, E, N, K, T, k, want_abssum=True)
    assert_matches_oracle(got, ref, ab, K // 32)
