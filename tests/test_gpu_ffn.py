"""A whole expert FFN on the GPU through the C ABI, every step in libftq:
quantise the tokens to Q8_1, first layer with the gated activation fused
(gate rows, then up rows), quantise its per-pair output to Q8_1, second layer
on those per-pair rows, router-weighted top-k combine ("Current Bug:
CuTeDSLMoERunner", Bug 6, the two-layer expert FFN with the first layer's
output as the second layer's per-pair input; FreeToken PR #185, Problem, the
activation that follows the first GEMV).

Each stage is checked against the oracle applied to the GPU's own output of
the stage before (so the bound of each stage is that stage's alone): the two
quantisations byte for byte, the layers within their fp32 bounds, the combine
within its fma-chain bound.  The whole chain is then captured in one HIP graph
and replayed, each replay bit-equal to the eager chain."""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_expert_quantize_amd import ftq, inputs
from tests._cases import U32, U64, assert_matches_oracle, gamma, say
from tests.test_gpu_act import assert_act_matches
from tests.test_gpu_down import _combine_bound

pytestmark = pytest.mark.gpu

PATHS = [ftq.PATH_GEMV, ftq.PATH_GROUPED, ftq.PATH_AUTO]
PATH_NAMES = {ftq.PATH_GEMV: "gemv", ftq.PATH_GROUPED: "grouped", ftq.PATH_AUTO: "auto"}


class Ffn:
    """Hidden size H, expert width I: w1 [E, 2I, H] (gate rows then up rows), w2 [E, H, I]."""

    def __init__(self, E, H, I, T, top_k, seed=0, kind="uniform", act=ftq.ACT_SILU):
        self.E, self.H, self.I, self.T, self.top_k, self.act = E, H, I, T, top_k, act
        self.w1 = inputs.weights(E, 2 * I, H, seed=seed)
        self.w2 = inputs.weights(E, H, I, seed=seed + 1)
        self.x = inputs.activations(T, H, seed=seed + 2)
        self.ids = inputs.routing(T, E, top_k, seed=seed, kind=kind)
        self.g = inputs.gates(T, top_k, seed=seed + 3)
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.dx, self.dids, self.dg = d(self.x), d(self.ids), d(self.g)
        self.dw1 = ftq.quantize_q4_0(d(self.w1))
        self.dw2 = ftq.quantize_q4_0(d(self.w2))
        P = T * top_k
        # every buffer of the chain, allocated once (the graph replays into them)
        self.aq = torch.empty(T * (H // 32) * 36, dtype=torch.uint8, device="cuda")
        self.h = torch.empty((P, I), dtype=torch.float32, device="cuda")
        self.hq = torch.empty(P * (I // 32) * 36, dtype=torch.uint8, device="cuda")
        self.y = torch.empty((P, H), dtype=torch.float32, device="cuda")
        self.out = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def workspaces(self, path):
        need1 = ftq.workspace_bytes(self.E, 2 * self.I, self.H, self.T, self.top_k, path)
        need2 = ftq.pairs_workspace_bytes(self.E, self.H, self.I, self.T, self.top_k, path)
        return (torch.empty(max(need1, 1), dtype=torch.uint8, device="cuda"),
                torch.empty(max(need2, 1), dtype=torch.uint8, device="cuda"))

    def chain(self, path, ws1, ws2):
        ftq.quantize_q8_1(self.dx, out=self.aq)
        ftq.moe_act(self.dw1, self.aq, self.dids, self.E, 2 * self.I, self.H, self.act,
                    path=path, out=self.h, workspace=ws1)
        ftq.quantize_q8_1(self.h, out=self.hq)
        ftq.moe_pairs(self.dw2, self.hq, self.dids, self.E, self.H, self.I,
                      path=path, out=self.y, workspace=ws2)
        ftq.combine_topk(self.y, self.dg, out=self.out)

    def snapshot(self):
        torch.cuda.synchronize()
        return {k: getattr(self, k).clone() for k in ("aq", "h", "hq", "y", "out")}


def check_stages(f: Ffn, s):
    """Each stage against the oracle on the GPU's input to that stage."""
    E, H, I, T, k = f.E, f.H, f.I, f.T, f.top_k
    ow1 = oracle.quantize_q4_0(f.w1).reshape(-1)
    ow2 = oracle.quantize_q4_0(f.w2).reshape(-1)
    assert np.array_equal(ftq_bytes(f.dw1), ow1) and np.array_equal(ftq_bytes(f.dw2), ow2)
    oa = oracle.quantize_q8_1(f.x).reshape(-1)
    assert np.array_equal(s["aq"].cpu().numpy(), oa), "token quantisation"
    # first layer: plain fp64 gate/up values, the activation applied in the check
    y1, ab1 = oracle.moe(ow1, oa, f.ids, E, 2 * I, H, T, k, want_abssum=True)
    h = s["h"].cpu().numpy()
    assert_act_matches(h, y1, ab1, H // 32, f.act)
    # the first layer's fp32 output, quantised per pair by each side
    ohq = oracle.quantize_q8_1(h).reshape(-1)
    assert np.array_equal(s["hq"].cpu().numpy(), ohq), "per-pair quantisation"
    # second layer on those per-pair rows
    y2, ab2 = oracle.moe(ow2, ohq, f.ids, E, H, I, T, k, want_abssum=True, per_pair=True)
    y = s["y"].cpu().numpy()
    assert_matches_oracle(y, y2, ab2, I // 32)
    # combine of the GPU's second-layer rows
    ref = oracle.combine_topk(y, f.g)
    got = s["out"].cpu().numpy()
    diff = np.abs(got.astype(np.float64) - ref)
    assert np.all(diff <= _combine_bound(f.g, y))
    if np.linalg.norm(ref) > 0:
        assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)


def ftq_bytes(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().reshape(-1)


# (E, H, I, T, top_k, routing)
SHAPES = {
    "tiny": (8, 256, 128, 16, 2, "uniform"),
    "ragged": (5, 96, 224, 11, 3, "uniform"),      # H/32 = 3 blocks, I = 224 not a tile multiple
    "zipf": (16, 512, 352, 150, 4, "zipf"),
}


@pytest.mark.parametrize("act", [ftq.ACT_SILU, ftq.ACT_GELU_TANH], ids=["silu", "gelu_tanh"])
@pytest.mark.parametrize("path", PATHS, ids=lambda p: PATH_NAMES[p])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_ffn_stages_match_oracle(shape, path, act):
    E, H, I, T, k, kind = SHAPES[shape]
    say(f"[ffn] {shape}: E={E} H={H} I={I} T={T} top_k={k} path={PATH_NAMES[path]} act={act}")
    f = Ffn(E, H, I, T, k, seed=41, kind=kind, act=act)
    ws1, ws2 = f.workspaces(path)
    f.chain(path, ws1, ws2)
    check_stages(f, f.snapshot())


@pytest.mark.parametrize("path", PATHS, ids=lambda p: PATH_NAMES[p])
def test_ffn_graph_replays_equal_eager(path):
    E, H, I, T, k, kind = SHAPES["zipf"]
    say(f"[ffn graph] E={E} H={H} I={I} T={T} top_k={k} path={PATH_NAMES[path]}")
    f = Ffn(E, H, I, T, k, seed=43, kind=kind, act=ftq.ACT_GELU_TANH)
    ws1, ws2 = f.workspaces(path)
    f.chain(path, ws1, ws2)
    eager = f.snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f.chain(path, ws1, ws2)              # warm up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f.chain(path, ws1, ws2)
    for i in range(3):
        for name in ("h", "y", "out"):
            getattr(f, name).fill_(float("nan"))
        f.aq.fill_(0xCD)
        f.hq.fill_(0xCD)
        ws1.fill_(0xAB)
        ws2.fill_(0xAB)
        g.replay()
        got = f.snapshot()
        for name, ref in eager.items():
            assert torch.equal(got[name], ref), f"replay {i}: {name} differs"
        _ = (eager["out"] * 2).sum().item()   # unrelated eager work between replays
