"""The pages' workloads at full size, in the launch configuration the benchmark
times (FTQ_PATH_AUTO): sampled output rows against the oracle, the over-cap
split-batch invariant bit for bit, and the pair-count boundary around 65535.

Workload shapes: FreeToken PR #185 "Performance" (nrows=1408, hidden=2816,
top_k=8, 128 experts; T = 2048/4096/8191) and "Test" (one token over the old
cap: 8192*8 = 65536 pairs, compared with the same batch split in half);
mlxcel PR #652 "Summary" (qwen3-30b-a3b at 8192 tokens, mixtral-8x7b at 32768
tokens)."""
import numpy as np
import pytest
import torch

from quantized_moe_expert_quantize_amd import ftq, inputs
from tests._cases import Case, assert_matches_oracle, sample_pairs, say

pytestmark = pytest.mark.gpu

_w_cache = {}


def _weights(E, N, K):
    key = (E, N, K)
    if key not in _w_cache:
        _w_cache.clear()
        _w_cache[key] = inputs.weights(E, N, K, seed=0)
    return _w_cache[key]


WORKLOADS = [
    # name, E, N, K, top_k, T, routing, sampled pairs
    ("page1_T2048", 128, 1408, 2816, 8, 2048, "uniform", 48),
    ("page1_T4096", 128, 1408, 2816, 8, 4096, "uniform", 48),
    ("page1_T8191", 128, 1408, 2816, 8, 8191, "uniform", 1024),
    ("page1_T1", 128, 1408, 2816, 8, 1, "uniform", 8),
    ("qwen3_up_T8192_zipf", 128, 768, 2048, 8, 8192, "zipf", 64),
    ("mixtral_T1", 8, 14336, 4096, 2, 1, "uniform", 2),
    ("mixtral_T8", 8, 14336, 4096, 2, 8, "uniform", 16),
    ("mixtral_T64", 8, 14336, 4096, 2, 64, "uniform", 12),
    ("mixtral_T32768", 8, 14336, 4096, 2, 32768, "uniform", 12),
]


@pytest.mark.parametrize("wl", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_workload_sampled_rows(wl):
    name, E, N, K, k, T, kind, ns = wl
    say(f"[workload] {name}: E={E} N={N} K={K} top_k={k} T={T} path={ftq.select_path(E, N, K, T, k)}")
    c = Case(E, N, K, T, k, seed=0, kind=kind, w32=_weights(E, N, K))
    c.assert_same_bytes()
    out = c.run()
    pairs = sample_pairs(T, k, ns, seed=1)
    got = out[torch.from_numpy(pairs).cuda()].cpu().numpy()
    del out
    ref, ab = c.oracle_out(pairs)
    assert_matches_oracle(got, ref, ab, c.nb)


def test_page1_T8191_every_pair_on_spread_rows():
    # all 65528 pairs of the bench workload, on 62 weight rows spread over N
    # (every 23rd, plus the last): the oracle runs on the experts' rows
    # restricted to those, which is the same arithmetic per output element
    E, N, K, k, T = 128, 1408, 2816, 8, 8191
    rows = np.unique(np.concatenate([np.arange(0, N, 23), [N - 1]]))
    c = Case(E, N, K, T, k, seed=0, w32=_weights(E, N, K))
    say(f"[workload] page-1 T={T}: all {T * k} pairs x {len(rows)} rows, path {ftq.select_path(E, N, K, T, k)}")
    got = c.run()[:, torch.from_numpy(rows).cuda()].cpu().numpy()
    sub = Case(E, len(rows), K, T, k, seed=0, w32=np.ascontiguousarray(_weights(E, N, K)[:, rows, :]),
               x32=c.x32, ids=c.ids)
    ref, ab = sub.oracle_out()
    assert_matches_oracle(got, ref, ab, c.nb)


@pytest.mark.parametrize("T", [8192, 16384])
@pytest.mark.parametrize("path", [ftq.PATH_AUTO, ftq.PATH_GROUPED, ftq.PATH_GEMV], ids=["auto", "grouped", "gemv"])
def test_over_cap_batch_equals_its_halves(T, path):
    E, N, K, k = 128, 1408, 2816, 8
    say(f"[over-cap] T={T} pairs={T * k} path={path}")
    c = Case(E, N, K, T, k, seed=0, w32=_weights(E, N, K))
    wq, aq, ids = c.gpu()
    full = ftq.moe(wq, aq, ids, E, N, K, path=path)
    h = T // 2
    nb36 = K // 32 * 36
    o1 = ftq.moe(wq, aq[:h], ids[:h], E, N, K, path=path)
    o2 = ftq.moe(wq, aq[h:], ids[h:], E, N, K, path=path)
    torch.cuda.synchronize()
    assert aq.shape[1] == nb36
    assert torch.equal(full[: h * k], o1) and torch.equal(full[h * k:], o2)
    # and the rows are right, not merely consistent
    pairs = sample_pairs(T, k, 16, seed=2)
    ref, ab = c.oracle_out(pairs)
    assert_matches_oracle(full[torch.from_numpy(pairs).cuda()].cpu().numpy(), ref, ab, c.nb)


@pytest.mark.parametrize("T", [65535, 65536, 65537])
def test_pair_count_around_the_old_grid_limit(T):
    E, N, K, k = 8, 64, 64, 1
    say(f"[boundary] pairs={T * k}")
    c = Case(E, N, K, T, k, seed=4)
    for path in (ftq.PATH_AUTO, ftq.PATH_GEMV, ftq.PATH_GROUPED):
        out = c.run(path)
        pairs = sample_pairs(T, k, 64, seed=3)
        ref, ab = c.oracle_out(pairs)
        assert_matches_oracle(out[torch.from_numpy(pairs).cuda()].cpu().numpy(), ref, ab, c.nb)
        wq, aq, ids = c.gpu()
        h = T // 2
        o1 = ftq.moe(wq, aq[:h], ids[:h], E, N, K, path=path)
        o2 = ftq.moe(wq, aq[h:], ids[h:], E, N, K, path=path)
        assert torch.equal(out, torch.cat([o1, o2]))
