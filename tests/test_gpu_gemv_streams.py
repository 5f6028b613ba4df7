"""The GEMV's per-pair-count streams give every pair the same bits.

The GEMV serves the pairs of one expert from one pass over its weight rows,
with a stream specialised for the number of pairs staged in the pass (1..8 for
plain Q4_0 rows whose K/32 is a multiple of 8, 1..4 otherwise, a guarded loop
for the rest).  Each pair's sum is the same fixed sequence of exact block dots,
scale FMAs and lane trees whatever the count (the exact per-block formulation
of the FreeToken PR #185 Q4_0 x Q8_1 GEMV, "Problem"), so a token routed to an
expert together with c - 1 others must get the bits it gets alone, for every c,
and the oracle's values within the stated bound.
"""
import numpy as np
import pytest
import torch

from quantized_moe_expert_quantize_amd import ftq
from tests._cases import Case, assert_matches_oracle, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [256, 2816, 96], ids=lambda k: f"K{k}")
def test_every_pair_count_gives_the_single_pair_bits(K):
    # one expert takes every pair (top_k = 1): c tokens stage c pairs in one
    # pass (two passes above 8); K = 256 and 2816 take the 16-byte loads and the
    # specialised streams, K = 96 (K/32 odd) the narrower loads
    E, N = 4, 72
    T = 12
    ids = np.zeros((T, 1), dtype=np.int32)
    c = Case(E, N, K, T, 1, seed=21, ids=ids)
    wq, aq, idd = c.gpu()
    nbytes = K // 32 * 36
    alone = []
    for t in range(T):
        a1 = aq.view(-1)[t * nbytes:(t + 1) * nbytes].contiguous()
        alone.append(ftq.moe(wq, a1, idd[:1].contiguous(), E, N, K, path=ftq.PATH_GEMV))
    alone = torch.cat(alone)
    for cnt in range(1, T + 1):
        say(f"[gemv streams] K={K}: {cnt} pairs on one expert")
        got = ftq.moe(wq, aq.view(-1)[: cnt * nbytes].contiguous(), idd[:cnt].contiguous(), E, N, K,
                      path=ftq.PATH_GEMV)
        assert torch.equal(got, alone[:cnt]), f"{cnt} pairs: a row differs from its single-pair bits"
    ref, ab = c.oracle_out()
    assert_matches_oracle(alone.cpu().numpy(), ref, ab, c.nb)
