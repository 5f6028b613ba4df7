"""GPU vs oracle parity through the C ABI: quantiser bytes bit-exact, integer
block partials bit-exact, fp32 outputs within the stated tolerance, for both
paths, on small shapes that span several tiles and ragged tails."""
import numpy as np
import pytest
import torch

from quantized_moe_expert_quantize_amd import ftq
from tests._cases import Case, assert_matches_oracle, say

pytestmark = pytest.mark.gpu

PATHS = [ftq.PATH_GEMV, ftq.PATH_GROUPED]
PATH_NAMES = {ftq.PATH_GEMV: "gemv", ftq.PATH_GROUPED: "grouped", ftq.PATH_AUTO: "auto"}

# (E, N, K, T, top_k, routing)
SHAPES = {
    "tiny": (8, 128, 256, 16, 2, "uniform"),               # the tiny workload
    "ragged_odd_nb": (4, 77, 96, 9, 3, "uniform"),         # K/32 = 3 (odd), N not a tile multiple
    "one_block": (3, 40, 32, 5, 1, "uniform"),             # K = 32
    "page1_rows": (16, 200, 2816, 33, 4, "uniform"),       # page-1 hidden size, ragged N
    "zipf": (32, 160, 512, 300, 8, "zipf"),                # skewed routing: hot and cold experts
    "many_pairs_per_expert": (4, 136, 384, 200, 2, "uniform"),
}


@pytest.fixture(scope="module", params=list(SHAPES))
def case(request):
    E, N, K, T, k, kind = SHAPES[request.param]
    say(f"[case] {request.param}: E={E} N={N} K={K} T={T} top_k={k} routing={kind}")
    return Case(E, N, K, T, k, seed=11, kind=kind)


def test_quantizers_bit_exact(case):
    case.assert_same_bytes()


@pytest.mark.parametrize("path", PATHS, ids=lambda p: PATH_NAMES[p])
def test_partials_bit_exact(case, path):
    got = case.partials(path)
    ref = case.oracle_partials()
    assert got.dtype == np.int32 and np.array_equal(got, ref)


@pytest.mark.parametrize("path", PATHS + [ftq.PATH_AUTO], ids=lambda p: PATH_NAMES[p])
def test_outputs_match_oracle(case, path):
    got = case.run(path).cpu().numpy()
    ref, ab = case.oracle_out()
    assert_matches_oracle(got, ref, ab, case.nb)


@pytest.mark.parametrize("path", PATHS, ids=lambda p: PATH_NAMES[p])
def test_deterministic(case, path):
    a = case.run(path).cpu().numpy()
    b = case.run(path).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_masked_and_duplicate_ids():
    E, N, K, T, k = 6, 96, 192, 40, 3
    ids = Case(E, N, K, T, k, seed=3).ids.copy()
    ids[0, 0] = -1
    ids[5, 2] = E
    ids[7, :] = 2**31 - 1
    ids[9, 1] = ids[9, 0]          # the same expert twice for one token
    c = Case(E, N, K, T, k, seed=3, ids=ids)
    ref, ab = c.oracle_out()
    for path in PATHS:
        got = c.run(path).cpu().numpy()
        assert_matches_oracle(got, ref, ab, c.nb)
        assert not got[0].any() and not got[5 * k + 2].any() and not got[7 * k:8 * k].any()
        assert np.array_equal(c.partials(path), c.oracle_partials())


@pytest.mark.parametrize("T", [40, 700])
def test_gemv_many_experts_skewed_counts(T):
    """More than 256 buckets (the GEMV's per-bucket cost prefix runs in several
    chunks), Zipf-skewed pair counts (the work split by cost gives hot experts
    more workgroups) and masked ids; T = 40 scans the ids in the kernel, T = 700
    (4200 pairs) reads the bucketed list."""
    E, N, K, k = 300, 48, 64, 6
    ids = Case(E, N, K, T, k, seed=4, kind="zipf").ids.copy()
    ids[1, 0] = -1
    ids[T - 1, k - 1] = E + 7
    c = Case(E, N, K, T, k, seed=4, ids=ids)
    counts = np.bincount(ids[(ids >= 0) & (ids < E)], minlength=E)
    say(f"[case] E={E} T={T}: routed experts {np.count_nonzero(counts)}, max pairs per expert {counts.max()}")
    ref, ab = c.oracle_out()
    got = c.run(ftq.PATH_GEMV).cpu().numpy()
    assert_matches_oracle(got, ref, ab, c.nb)
    assert not got[1 * k].any() and not got[T * k - 1].any()
    assert np.array_equal(c.partials(ftq.PATH_GEMV), c.oracle_partials())


def test_most_experts_supported():
    """E = 4095, the largest expert count the bucket tables take (one pair per
    expert at most here); both paths, against the oracle."""
    E, N, K, T, k = 4095, 40, 64, 24, 3
    ids = Case(E, N, K, T, k, seed=9).ids.copy()
    ids[0, 0] = E - 1
    ids[2, 1] = -3
    c = Case(E, N, K, T, k, seed=9, ids=ids)
    ref, ab = c.oracle_out()
    for path in PATHS:
        assert_matches_oracle(c.run(path).cpu().numpy(), ref, ab, c.nb)
        assert np.array_equal(c.partials(path), c.oracle_partials())


def test_all_ids_masked_gives_zeros():
    E, N, K, T, k = 4, 64, 64, 20, 2
    c = Case(E, N, K, T, k, ids=np.full((T, k), -5, np.int32))
    for path in PATHS:
        out = c.run(path)
        assert not out.any()


def test_single_expert_dense_case():
    c = Case(1, 300, 640, 70, 1, seed=5)
    ref, ab = c.oracle_out()
    for path in PATHS:
        assert_matches_oracle(c.run(path).cpu().numpy(), ref, ab, c.nb)


def test_zero_tokens_writes_nothing():
    c = Case(4, 32, 64, 0, 2)
    wq, aq, ids = c.gpu()
    out = torch.full((0, 32), 7.0, device="cuda")
    ftq.moe(wq, aq, ids, 4, 32, 64, out=out)
    torch.cuda.synchronize()


def test_quantize_q8_1_closed_forms():
    x = np.zeros((3, 64), np.float32)
    x[1, :32] = 0.25                           # constant block -> all codes 127
    x[2, 0] = 127.0                            # d = 1: ties round away from zero
    x[2, 1:7] = [2.5, -2.5, 0.5, -0.5, 126.5, -3.5]
    x[2, 40] = -1e-30                          # tiny single value -> -127 with a subnormal-free d
    got = ftq.quantize_q8_1(torch.from_numpy(x).cuda()).cpu().numpy()
    import oracle
    assert np.array_equal(got, oracle.quantize_q8_1(x))
    q = got.reshape(3, 2, 36)[..., 4:].view(np.int8)
    assert not got[0].any()
    assert np.all(q[1, 0] == 127)
    assert q[2, 0, :7].tolist() == [127, 3, -3, 1, -1, 127, -4]


def test_quantize_q8_1_many_rows_and_ragged():
    for T, K in ((1, 4096), (37, 2816), (1000, 2048), (3, 32)):
        x = np.random.default_rng(T).standard_normal((T, K)).astype(np.float32) * np.float32(3.0)
        import oracle
        got = ftq.quantize_q8_1(torch.from_numpy(x).cuda()).cpu().numpy()
        assert np.array_equal(got, oracle.quantize_q8_1(x)), (T, K)


def _near_tie_blocks():
    """Blocks whose x/d falls on or within a few ulps of a rounding boundary
    k + 1/2, for exact and inexact d, and blocks whose d lies outside
    [2^-100, 2^100] or is subnormal: every place where a quotient formed from a
    reciprocal could round to a different code than the correctly rounded
    division."""
    f32 = np.float32
    rows = []
    for amax in (127.0, 1.0, 3.0, 0.3, 1e-3, 7.77e5, 1e-28, 1e32, 1e-32, 1e33, 1e-38, 1e-40):
        amax = f32(amax)
        d = f32(amax / f32(127.0))
        for k0 in (0, 30, 60, 90, 120):
            vals = [amax]
            for k in range(k0, k0 + 6):
                c = f32(f32(k + 0.5) * d)
                for step in (-2, -1, 0, 1, 2):
                    v = c
                    for _ in range(abs(step)):
                        v = np.nextafter(v, f32(np.inf) if step > 0 else f32(-np.inf))
                    if abs(v) <= amax:
                        vals.append(v if (k + step) % 2 == 0 else -v)
            block = np.zeros(32, f32)
            vals = vals[:32]
            block[:len(vals)] = vals
            rows.append(block)
    return np.stack(rows)


def test_quantize_q8_1_near_ties():
    import oracle
    x = _near_tie_blocks()
    got = ftq.quantize_q8_1(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.quantize_q8_1(x))


def _double_rounding_blocks(n=1 << 20, seed=77):
    """Seeded search (host only) for Q8_1 blocks whose s = d*sum(q) rounds
    differently when taken to fp16 in one step than via fp32.  The oracle holds
    the expected bytes; this only finds inputs where a fused conversion would
    show."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, 32)) * rng.choice([0.01, 1, 30, 500], size=(n, 1))).astype(np.float32)
    d = (np.abs(x).max(1) / np.float32(127)).astype(np.float32)
    r = x / d[:, None]
    q = np.where(r >= 0, np.floor(r + np.float32(0.5)), np.ceil(r - np.float32(0.5))).astype(np.int64)
    S = q.sum(1)
    once = (d.astype(np.float64) * S).astype(np.float16).view(np.uint16)
    twice = (d * S.astype(np.float32)).astype(np.float16).view(np.uint16)
    return x[np.nonzero(once != twice)[0]]


def test_quantize_q8_1_sum_rounds_via_fp32():
    import oracle
    x = _double_rounding_blocks()
    assert len(x) >= 16
    x = np.ascontiguousarray(x.reshape(-1, 32))
    got = ftq.quantize_q8_1(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.quantize_q8_1(x))


def test_launch_check_reports_geometry_and_does_not_latch():
    c = Case(8, 128, 256, 16, 2)
    wq, aq, ids = c.gpu()
    good = c.run(ftq.PATH_GEMV)
    L = ftq.lib()
    L.ftq_debug_force_block_threads(4096)
    try:
        with pytest.raises(ftq.FtqError) as ei:
            ftq.moe(wq, aq, ids, 8, 128, 256, path=ftq.PATH_GEMV)
        assert ei.value.status == ftq.ERR_LAUNCH
        msg = str(ei.value)
        assert "moe_gemv_kernel" in msg and "block=(4096" in msg and "grid=(" in msg and "lds=" in msg
    finally:
        L.ftq_debug_force_block_threads(0)
    again = c.run(ftq.PATH_GEMV)
    assert torch.equal(again, good)


def test_graph_capture_and_replay():
    c = Case(16, 256, 512, 96, 4, seed=2)
    wq, aq, ids = c.gpu()
    for path in PATHS:
        eager = c.run(path).clone()
        out = torch.empty_like(eager)
        need = ftq.workspace_bytes(16, 256, 512, 96, 4, path)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            ftq.moe(wq, aq, ids, 16, 256, 512, path=path, out=out, workspace=ws)   # warm up on the side stream
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ftq.moe(wq, aq, ids, 16, 256, 512, path=path, out=out, workspace=ws)
        for i in range(4):
            out.fill_(float("nan"))
            ws.fill_(0xAB)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {i} differs"
            _ = (eager * 2).sum().item()      # unrelated eager work between replays


@pytest.mark.parametrize("path", PATHS + [ftq.PATH_AUTO], ids=lambda p: PATH_NAMES[p])
def test_route_then_routed_equals_one_call(path):
    c = Case(16, 200, 512, 150, 4, seed=8, kind="zipf")
    wq, aq, ids = c.gpu()
    one = c.run(path)
    need = ftq.workspace_bytes(16, 200, 512, 150, 4, path)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    ftq.moe_route(ids, 16, ws, path)
    out = torch.empty_like(one)
    ftq.moe_routed(wq, aq, ids, 16, 200, 512, out, ws, path)
    # a second matmul over the same routing (another weight set, same pairs)
    w2 = ftq.quantize_q4_0(torch.from_numpy(c.w32[::-1].copy()).cuda())
    out2 = torch.empty_like(one)
    ftq.moe_routed(w2, aq, ids, 16, 200, 512, out2, ws, path)
    ref2 = ftq.moe(w2, aq, ids, 16, 200, 512, path=path)
    torch.cuda.synchronize()
    assert torch.equal(out, one) and torch.equal(out2, ref2)


def test_wide_offset_variant_matches():
    """The 64-bit-offset tile kernels (used past 4 GiB of staged activations) are
    forced on small cases in a child process and must match the oracle: the
    int8, fp16 and warp-specialised Q4_0 kernels and the Q4_1 / Q8_0 kernels."""
    import os
    import subprocess
    import sys
    code = (
        "import numpy as np\n"
        "from tests._cases import Case, assert_matches_oracle\n"
        "from quantized_moe_expert_quantize_amd import ftq\n"
        "from tests.test_gpu_gguf import WCase\n"
        "c = Case(8, 200, 640, 120, 4, seed=6)\n"
        "ref, ab = c.oracle_out()\n"
        "refp = c.oracle_partials()\n"
        "for v in (ftq.GROUPED_I8, ftq.GROUPED_F16, ftq.GROUPED_F16_WS):\n"
        "    ftq.grouped_kernel(v)\n"
        "    assert_matches_oracle(c.run(ftq.PATH_GROUPED).cpu().numpy(), ref, ab, c.nb)\n"
        "    assert np.array_equal(c.partials(ftq.PATH_GROUPED), refp)\n"
        "ftq.grouped_kernel(ftq.GROUPED_I8)\n"
        "for wt in (ftq.W_Q4_1, ftq.W_Q8_0):\n"
        "    w = WCase(wt, 8, 96, 640, 120, 4, seed=7)\n"
        "    assert np.array_equal(w.partials(ftq.PATH_GROUPED), w.oracle_partials())\n"
        "    w.check(w.run(ftq.PATH_GROUPED))\n"
        "print('wide ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, FTQ_FORCE_WIDE="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "wide ok" in r.stdout, r.stdout + r.stderr


def test_binding_rejects_wrong_out_size():
    """A caller's out buffer of the wrong size is refused before any launch."""
    c = Case(4, 32, 64, 3, 2)
    wq, aq, ids = c.gpu()
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="out must hold"):
        ftq.moe(wq, aq, ids, 4, 32, 64, out=f32(5, 32))
    with pytest.raises(ValueError, match="out must hold"):
        ftq.moe_act(wq, aq, ids, 4, 32, 64, ftq.ACT_SILU, out=f32(6, 32))
    with pytest.raises(ValueError, match="out must hold"):
        ftq.quantize_q8_1(f32(3, 64), out=torch.empty(10, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError, match="out must hold"):
        ftq.combine_topk(f32(6, 8), f32(3, 2), out=f32(3, 7))
    torch.cuda.synchronize()
