"""Routing tables: the one-workgroup bucketing and the three-kernel bucketing
build the same tables, and both equal the tables computed on the host.

The grouped path sorts the flat (token, top-k) pairs by routed expert: each
expert's pairs form one contiguous segment in ascending pair order, preceded by
the per-expert segment offsets (with the leading 0 and the total) and followed
by the per-expert tile counts and one descriptor per tile (the expert-sorted
layout of "Current Bug: CuTeDSLMoERunner", Key Architecture and Bug 4; masked
ids, outside [0, E), form one more bucket, Bug 8).  The host side here is a
stable sort of the pair ids by bucket.
"""
import numpy as np
import pytest
import torch

from quantized_moe_expert_quantize_amd import ftq, inputs
from tests._cases import say

pytestmark = pytest.mark.gpu

CHUNK = 1024


def _align(v):
    return (v + 255) // 256 * 256


def _tile_m(E, T, k):
    per_expert = T * k // E
    return 128 if per_expert >= 96 else 64 if per_expert >= 40 else 32


def _layout(E, T, k):
    pairs, buckets = T * k, E + 1
    chunks = (pairs + CHUNK - 1) // CHUNK
    tm = _tile_m(E, T, k)
    off = _align(4 * chunks * buckets)
    lay = {"offsets": off}
    off = _align(off + 4 * (buckets + 1))
    lay["tiles"] = off
    off = _align(off + 4 * (buckets + 1))
    lay["sorted"] = off
    off = _align(off + 4 * pairs)
    lay["tdesc"] = off
    lay["max_tiles"] = (pairs + buckets * (tm - 1)) // tm
    lay["tm"] = tm
    return lay


def _host_tables(ids, E, tm):
    flat = ids.reshape(-1)
    bucket = np.where((flat >= 0) & (flat < E), flat, E).astype(np.int64)
    counts = np.bincount(bucket, minlength=E + 1)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.argsort(bucket, kind="stable").astype(np.int32)
    ntiles = (counts + tm - 1) // tm
    tiles = np.concatenate([[0], np.cumsum(ntiles)]).astype(np.int32)
    desc = []
    for b in range(E + 1):
        for t in range(int(ntiles[b])):
            slot0 = int(offsets[b]) + t * tm
            desc.append((b, slot0, min(tm, int(offsets[b + 1]) - slot0), 0))
    return offsets, tiles, order, np.array(desc, dtype=np.int32).reshape(-1, 4)


def _route(ids_d, E, need, split):
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ftq.route_kernels(split)
    try:
        ftq.moe_route(ids_d, E, ws, ftq.PATH_GROUPED)
    finally:
        ftq.route_kernels(False)
    torch.cuda.synchronize()
    return ws.cpu().numpy()


# (E, T, top_k, routing, masked): one chunk, ragged chunks, the 8-chunk limit
# of the one-workgroup bucketing, one pair over it, Zipf routing, many experts
# (up to the 2048-bucket limit and past it)
CASES = [
    (8, 100, 2, "uniform", False),
    (128, 64, 8, "uniform", False),
    (128, 2000, 8, "uniform", True),
    (128, 1024, 8, "uniform", False),
    (128, 1025, 8, "uniform", False),
    (32, 2000, 4, "zipf", True),
    (1024, 700, 4, "uniform", False),
    (2047, 1024, 4, "uniform", True),
    (4000, 300, 8, "uniform", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "E{}T{}k{}{}{}".format(c[0], c[1], c[2], c[3], "m" if c[4] else ""))
def test_one_workgroup_route_equals_three_kernels_and_host(case):
    E, T, k, kind, masked = case
    say(f"[route] E={E} T={T} top_k={k} {kind} masked={masked}")
    ids = inputs.routing(T, E, k, seed=E + T, kind=kind)
    if masked:
        ids[::7, 0] = -1
        ids[3::11, -1] = E + 5
    ids_d = torch.from_numpy(ids).cuda()
    need = ftq.workspace_bytes(E, 64, 256, T, k, ftq.PATH_GROUPED)
    lay = _layout(E, T, k)
    one = _route(ids_d, E, need, False)
    three = _route(ids_d, E, need, True)
    start = lay["offsets"]
    assert np.array_equal(one[start:], three[start:]), "the two bucketings' tables differ"
    offsets, tiles, order, desc = _host_tables(ids, E, lay["tm"])
    nb = E + 1

    def i32(at, n):
        return one[at: at + 4 * n].view(np.int32)

    assert np.array_equal(i32(lay["offsets"], nb + 1), offsets)
    assert np.array_equal(i32(lay["tiles"], nb + 1), tiles)
    assert np.array_equal(i32(lay["sorted"], T * k), order)
    assert len(desc) <= lay["max_tiles"]
    assert np.array_equal(i32(lay["tdesc"], 4 * len(desc)).reshape(-1, 4), desc)
