"""Pins of the CPU oracle against facts that do not come from the oracle itself:
numpy's IEEE float16 conversion, exact rational arithmetic, closed forms of the
quantisers on inputs that already lie on the quantisation grid, textbook dense
matmul, integer einsum, Higham's summation bound, and the invariants the pages
state (split batch equals the halves; masked experts give zero rows)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from quantized_moe_expert_quantize_amd import inputs
from tests import _decode

U64 = 2.0 ** -53          # unit roundoff of fp64


def gamma(n, u):
    return n * u / (1 - n * u)


# ---------------------------------------------------------------- fp16 -----

def test_fp16_decode_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_fp32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _fp16_edges():
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, -65520.0, 65536.0, 1e30, -1e30,
         2.0 ** -14, 2.0 ** -24, 2.0 ** -25, -2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
         3 * 2.0 ** -25, 5 * 2.0 ** -25, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -14 - 2.0 ** -24,
         1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -23, 2049.0, 2051.0,
         np.inf, -np.inf, 1.0 / 127.0, 4064.0 / 127.0]
    return np.array(v, dtype=np.float32)


def test_fp16_encode_edges_and_random():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    rand_any = bits.view(np.float32)
    rand_range = (rng.standard_normal(1_000_000) * rng.choice([1e-6, 1e-3, 1.0, 1e3, 3e4], 1_000_000)).astype(np.float32)
    # values exactly halfway between neighbouring fp16 numbers (ties-to-even cases)
    h = rng.integers(0, 0x7bff, size=100_000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    for f in (_fp16_edges(), rand_any, rand_range, ties):
        got = oracle.fp32_to_fp16(f)
        with np.errstate(over="ignore"):
            ref = f.astype(np.float16).view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.all(np.isnan(got[nan].view(np.float16)))


# ---------------------------------------------------------------- Q8_1 -----

def test_q8_1_zero_block():
    y = oracle.quantize_q8_1(np.zeros((2, 64), np.float32))
    assert not y.any()


def test_q8_1_constant_block():
    for c in (0.5, -3.25, 1e-3):
        y = oracle.quantize_q8_1(np.full((1, 32), c, np.float32))
        d, s, q = _decode.q8_1(y, 32)
        assert np.all(q == (127 if c > 0 else -127))
        assert d[0, 0] == np.float16(np.float32(abs(c)) / np.float32(127))
        assert s[0, 0] == np.float16(np.float32(np.float32(abs(c)) / np.float32(127)) * np.float32(q.sum()))


def test_q8_1_single_nonzero():
    x = np.zeros((1, 32), np.float32)
    x[0, 7] = -0.3
    _, _, q = _decode.q8_1(oracle.quantize_q8_1(x), 32)
    assert q[0, 0, 7] == -127 and np.count_nonzero(q) == 1


def test_q8_1_exact_grid_recovery():
    """Inputs q*2^j with an element of magnitude 127 quantise back to exactly q, d = 2^j."""
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, size=(64, 32))
    q[np.arange(64), rng.integers(0, 32, 64)] = rng.choice([-127, 127], 64)
    j = rng.integers(-20, 4, size=(64, 1))
    x = (q * np.exp2(j)).astype(np.float32)
    y = oracle.quantize_q8_1(x.reshape(8, 256))
    d, s, qq = _decode.q8_1(y, 256)
    assert np.array_equal(qq.reshape(64, 32), q)
    assert np.array_equal(d.reshape(64), np.exp2(j[:, 0]))
    # s = fp16(d * sum q): d*sum is exact here, so numpy's own float16 gives the answer
    assert np.array_equal(s.reshape(64), (np.exp2(j[:, 0]) * q.sum(1)).astype(np.float16).astype(np.float64))


def test_q8_1_rounding_is_half_away_from_zero():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0           # amax = 127 -> d = 1 exactly
    x[0, 1:9] = [2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -3.5]
    _, _, q = _decode.q8_1(oracle.quantize_q8_1(x), 32)
    assert q[0, 0, :9].tolist() == [127, 3, -3, 1, -1, 2, -2, 127, -4]


def test_q8_1_random_properties():
    x = inputs.activations(64, 2816, seed=3)
    d, s, q = _decode.q8_1(oracle.quantize_q8_1(x), 2816)
    xb = x.reshape(64, 88, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.abs(q).max(-1) == 127)                       # the amax element maps to +-127
    # half a step, widened by the fp32 rounding of x/d (|x/d| <= 127)
    assert np.all(np.abs(xb - q * d32[..., None]) <= (0.5 + 128 * 2.0 ** -23) * d32[..., None])
    assert np.all(np.sign(q) * np.sign(xb) >= 0)
    assert np.array_equal(d, d32.astype(np.float32).astype(np.float16).astype(np.float64))


# ---------------------------------------------------------------- Q4_0 -----

def test_q4_0_exact_grid_recovery():
    """(c) * d with codes c in [-8, 7] and one c = -8 quantise back to q = c + 8 and d."""
    rng = np.random.default_rng(9)
    c = rng.integers(-7, 8, size=(100, 32))
    c[np.arange(100), rng.integers(0, 32, 100)] = -8
    d = rng.choice([-1, 1], size=(100, 1)) * np.exp2(rng.integers(-14, 2, size=(100, 1)).astype(np.float64))
    x = (c * d).astype(np.float32)
    dd, qq = _decode.q4_0(oracle.quantize_q4_0(x.reshape(25, 128)), 128)
    assert np.array_equal(qq.reshape(100, 32), c)
    assert np.array_equal(dd.reshape(100), d[:, 0])


def test_q4_0_nibble_order_and_clamp():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = -8.0               # max magnitude, negative -> d = 1
    x[0, 1] = 7.0
    x[0, 16] = 3.0               # high nibble of byte 0
    x[0, 17] = -1.0
    y = oracle.quantize_q4_0(x)
    assert y[0, 0:2].view(np.float16)[0] == 1.0
    assert y[0, 2] == (0 | (11 << 4))        # elements 0 and 16
    assert y[0, 3] == (15 | (7 << 4))        # elements 1 and 17
    # positive maximum: d is negative and the value -m maps past 7 -> clamped to 15
    x2 = np.zeros((1, 32), np.float32)
    x2[0, 3] = 4.0
    x2[0, 4] = -4.0
    d2, q2 = _decode.q4_0(oracle.quantize_q4_0(x2), 32)
    assert d2[0, 0] == -0.5 and q2[0, 0, 3] == -8 and q2[0, 0, 4] == 7
    # all-zero block: d = 0, every code 8 (value 0)
    d3, q3 = _decode.q4_0(oracle.quantize_q4_0(np.zeros((1, 32), np.float32)), 32)
    assert d3[0, 0] == 0 and np.all(q3 == 0)


def test_q4_0_random_error_bound():
    w = inputs.weights(2, 16, 256, seed=1).reshape(32, 256)
    d, q = _decode.q4_0(oracle.quantize_q4_0(w), 256)
    xb = w.reshape(32, 8, 32).astype(np.float64)
    ad = np.abs(d)[..., None]
    # half a step, except at the clamped top code 7 (x/d may reach 8), plus the fp16
    # rounding of d (|q| <= 8) and the fp32 rounding of x/d
    step = np.where(q == 7, 1.0, 0.5 + 8 * 2.0 ** -23)
    assert np.all(np.abs(xb - q * d[..., None]) <= step * ad + 8 * ad * 2.0 ** -11)
    assert np.all(np.abs(q).max(-1) == 8)               # the max-magnitude element has code 0


# ---------------------------------------------------------------- MoE ------

def _tiny(seed=0, E=8, top_k=2, T=16, K=256, N=128, kind="uniform"):
    w = oracle.quantize_q4_0(inputs.weights(E, N, K, seed=seed))
    a = oracle.quantize_q8_1(inputs.activations(T, K, seed=seed))
    ids = inputs.routing(T, E, top_k, seed=seed, kind=kind)
    return w, a, ids, dict(E=E, N=N, K=K, T=T, top_k=top_k)


def _run(w, a, ids, c, **kw):
    return oracle.moe(w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"], **kw)


def test_moe_exact_rational_bruteforce():
    """Exact value with Fractions; the oracle's fp64 error is within gamma_nb * sum|term|."""
    w, a, ids, c = _tiny(E=3, top_k=2, T=3, K=96, N=5)
    out, ab = _run(w, a, ids, c, want_abssum=True)
    wd, wq = _decode.q4_0(w.reshape(3, 5, -1), 96)
    ad, _, aq = _decode.q8_1(a, 96)
    nb = 3
    for p in range(c["T"] * c["top_k"]):
        t, e = p // 2, int(ids.reshape(-1)[p])
        for n in range(5):
            exact = Fraction(0)
            for b in range(nb):
                P = sum(int(wq[e, n, b, i]) * int(aq[t, b, i]) for i in range(32))
                exact += Fraction(P) * Fraction(wd[e, n, b]) * Fraction(ad[t, b])
            err = abs(Fraction(out[p, n]) - exact)
            assert err <= Fraction(gamma(nb, U64)) * Fraction(ab[p, n])


def test_moe_dense_special_case_matches_numpy_matmul():
    """E = 1, top_k = 1 reduces the MoE to a dense dequantise-then-matmul."""
    w, a, ids, c = _tiny(E=1, top_k=1, T=9, K=320, N=33)
    out, ab = _run(w, a, ids, c, want_abssum=True)
    wd, wq = _decode.q4_0(w.reshape(33, -1), 320)
    ad, _, aq = _decode.q8_1(a, 320)
    Wf = (wq * wd[..., None]).reshape(33, 320)
    Af = (aq * ad[..., None]).reshape(9, 320)
    ref = Af @ Wf.T
    # both sides round only in fp64 sums; numpy's blocked sum is bounded the same way
    bound = 2 * gamma(320, U64) * (np.abs(Af) @ np.abs(Wf).T)
    assert np.all(np.abs(out - ref) <= bound)


def test_moe_partials_match_integer_einsum():
    w, a, ids, c = _tiny()
    P = oracle.moe_partials(w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"])
    _, wq = _decode.q4_0(w.reshape(c["E"], c["N"], -1), c["K"])
    _, _, aq = _decode.q8_1(a, c["K"])
    tok = np.arange(c["T"] * c["top_k"]) // c["top_k"]
    ref = np.einsum("pnbi,pbi->pnb", wq[ids.reshape(-1)], aq[tok])
    assert P.dtype == np.int32 and np.array_equal(P, ref)
    assert np.abs(P).max() <= 8 * 127 * 32


def test_moe_outputs_equal_scaled_partials_sum():
    w, a, ids, c = _tiny(seed=4)
    out = _run(w, a, ids, c)
    P = oracle.moe_partials(w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"]).astype(np.float64)
    wd, _ = _decode.q4_0(w.reshape(c["E"], c["N"], -1), c["K"])
    ad, _, _ = _decode.q8_1(a, c["K"])
    tok = np.arange(c["T"] * c["top_k"]) // c["top_k"]
    terms = P * wd[ids.reshape(-1)] * ad[tok][:, None, :]
    ref = terms.sum(-1)
    assert np.all(np.abs(out - ref) <= 2 * gamma(8, U64) * np.abs(terms).sum(-1))


def test_moe_closed_forms():
    E, N, K, T, k = 2, 3, 64, 2, 1
    nb = K // 32
    # all weight codes 8 -> every output exactly zero
    w = np.zeros((E, N, nb, 18), np.uint8)
    w[..., 0:2] = np.frombuffer(np.float16(0.75).tobytes(), np.uint8)
    w[..., 2:] = 0x88
    a = oracle.quantize_q8_1(inputs.activations(T, K, seed=2))
    ids = np.array([[1], [0]], np.int32)
    assert not oracle.moe(w.reshape(-1), a, ids, E, N, K, T, k).any()
    # one nonzero weight code against a one-hot activation: out = d4*d8*(q4-8)*q8
    w2 = w.copy()
    w2[1, 2, 1, 2 + 5] = 0x80 | 13                      # element 5 of block 1 -> code 13 (value 5)
    x = np.zeros((T, K), np.float32)
    x[0, 32 + 5] = -2.0                                 # block 1, element 5 -> q = -127
    a2 = oracle.quantize_q8_1(x)
    out = oracle.moe(w2.reshape(-1), a2, ids, E, N, K, T, k)
    d8 = float(np.float16(np.float32(2.0) / np.float32(127)))
    expect = np.zeros((T * k, N))
    expect[0, 2] = 0.75 * d8 * 5 * -127
    assert np.array_equal(out, expect)


def test_moe_masked_and_duplicate_ids():
    w, a, ids, c = _tiny()
    bad = ids.copy()
    bad[0, 0] = -1
    bad[3, 1] = c["E"]
    bad[5, 1] = bad[5, 0]                               # duplicate expert within a token
    out = _run(w, a, bad, c)
    ref = _run(w, a, ids, c)
    assert not out[0].any() and not out[3 * 2 + 1].any()
    assert np.array_equal(out[5 * 2 + 1], out[5 * 2 + 0])
    keep = np.ones(out.shape[0], bool)
    keep[[0, 7, 11]] = False
    assert np.array_equal(out[keep], ref[keep])


def test_moe_split_batch_equals_halves():
    """A batch equals the same batch computed as two halves [FreeToken PR #185, "Test"]."""
    w, a, ids, c = _tiny(T=17)
    full = _run(w, a, ids, c)
    nb36 = c["K"] // 32 * 36
    h = 9
    c1 = dict(c, T=h)
    c2 = dict(c, T=c["T"] - h)
    a_ = a.reshape(c["T"], nb36)
    o1 = _run(w, np.ascontiguousarray(a_[:h]).reshape(-1), np.ascontiguousarray(ids[:h]), c1)
    o2 = _run(w, np.ascontiguousarray(a_[h:]).reshape(-1), np.ascontiguousarray(ids[h:]), c2)
    assert np.array_equal(full, np.concatenate([o1, o2]))


def test_moe_token_permutation_and_expert_relabel():
    w, a, ids, c = _tiny(seed=7)
    out = _run(w, a, ids, c)
    rng = np.random.default_rng(0)
    perm = rng.permutation(c["T"])
    nb36 = c["K"] // 32 * 36
    a_p = np.ascontiguousarray(a.reshape(c["T"], nb36)[perm]).reshape(-1)
    out_p = _run(w, a_p, np.ascontiguousarray(ids[perm]), c)
    assert np.array_equal(out_p.reshape(c["T"], c["top_k"], -1), out.reshape(c["T"], c["top_k"], -1)[perm])
    relabel = rng.permutation(c["E"])                   # new id of old expert e is relabel[e]
    w_r = np.empty_like(w.reshape(c["E"], -1))
    w_r[relabel] = w.reshape(c["E"], -1)
    out_r = _run(np.ascontiguousarray(w_r).reshape(-1), a, np.ascontiguousarray(relabel[ids]).astype(np.int32), c)
    assert np.array_equal(out_r, out)


def test_moe_pairs_matches_full():
    w, a, ids, c = _tiny(seed=2, kind="zipf")
    full, ab = _run(w, a, ids, c, want_abssum=True)
    pairs = np.array([0, 5, 31, 17, 5], np.int64)
    sub, sab = oracle.moe_pairs(w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"], pairs, want_abssum=True)
    assert np.array_equal(sub, full[pairs]) and np.array_equal(sab, ab[pairs])


def test_routing_generators():
    u = inputs.routing(4096, 128, 8, seed=0)
    assert u.shape == (4096, 8) and u.min() >= 0 and u.max() < 128
    assert all(len(set(r)) == 8 for r in u[:512].tolist())
    z = inputs.routing(8192, 128, 8, seed=0, kind="zipf")
    counts = np.bincount(z.reshape(-1), minlength=128)
    assert all(len(set(r)) == 8 for r in z[:512].tolist())
    assert counts[0] > 20 * counts[-1]                 # hot and cold experts
    assert np.array_equal(inputs.routing(4096, 128, 8, seed=0), u)


# ------------------------------------------- second layer: per-pair rows ------

def _tiny_pp(seed=0, E=8, top_k=2, T=16, K=256, N=128, kind="uniform"):
    """Per-pair activations: one distinct Q8_1 row per (token, slot) pair."""
    w = oracle.quantize_q4_0(inputs.weights(E, N, K, seed=seed))
    a = oracle.quantize_q8_1(inputs.activations(T * top_k, K, seed=seed + 101))
    ids = inputs.routing(T, E, top_k, seed=seed, kind=kind)
    return w, a, ids, dict(E=E, N=N, K=K, T=T, top_k=top_k)


def test_moe_per_pair_exact_rational_bruteforce():
    """Pair p reads activation row p (not p // top_k): exact Fractions, fp64 error bound."""
    w, a, ids, c = _tiny_pp(E=3, top_k=3, T=2, K=96, N=4, seed=3)
    out, ab = _run(w, a, ids, c, want_abssum=True, per_pair=True)
    wd, wq = _decode.q4_0(w.reshape(3, 4, -1), 96)
    ad, _, aq = _decode.q8_1(a, 96)
    for p in range(6):
        e = int(ids.reshape(-1)[p])
        for n in range(4):
            exact = Fraction(0)
            for b in range(3):
                P = sum(int(wq[e, n, b, i]) * int(aq[p, b, i]) for i in range(32))
                exact += Fraction(P) * Fraction(wd[e, n, b]) * Fraction(ad[p, b])
            assert abs(Fraction(out[p, n]) - exact) <= Fraction(gamma(3, U64)) * Fraction(ab[p, n])


def test_moe_per_pair_partials_match_integer_einsum():
    w, a, ids, c = _tiny_pp(seed=5, kind="zipf")
    P = oracle.moe_partials(w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"], per_pair=True)
    _, wq = _decode.q4_0(w.reshape(c["E"], c["N"], -1), c["K"])
    _, _, aq = _decode.q8_1(a, c["K"])
    ref = np.einsum("pnbi,pbi->pnb", wq[ids.reshape(-1)], aq)
    assert P.dtype == np.int32 and np.array_equal(P, ref)


def test_moe_per_pair_replicated_rows_equal_per_token():
    """Per-pair rows that repeat each token's row give the per-token result exactly."""
    w, a, ids, c = _tiny(seed=6)
    nb36 = c["K"] // 32 * 36
    a_rep = np.ascontiguousarray(np.repeat(a.reshape(c["T"], nb36), c["top_k"], axis=0)).reshape(-1)
    assert np.array_equal(_run(w, a_rep, ids, c, per_pair=True), _run(w, a, ids, c))
    pairs = np.array([3, 0, 31, 3], np.int64)
    sub = oracle.moe_pairs(w, a_rep, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"], pairs, per_pair=True)
    assert np.array_equal(sub, _run(w, a, ids, c)[pairs])


def test_moe_per_pair_masked_rows_zero():
    w, a, ids, c = _tiny_pp(seed=8)
    bad = ids.copy()
    bad[2, 1] = -5
    bad[7, 0] = c["E"] + 3
    out = _run(w, a, bad, c, per_pair=True)
    ref = _run(w, a, ids, c, per_pair=True)
    assert not out[5].any() and not out[14].any()
    keep = np.ones(out.shape[0], bool)
    keep[[5, 14]] = False
    assert np.array_equal(out[keep], ref[keep])


def test_combine_topk_bruteforce_and_special_cases():
    rng = np.random.default_rng(11)
    T, k, N = 7, 3, 45
    y = rng.standard_normal((T * k, N))
    g = rng.random((T, k)).astype(np.float32)
    out, ab = oracle.combine_topk(y, g, want_abssum=True)
    exact = [[sum(Fraction(float(g[t, j])) * Fraction(y[t * k + j, n]) for j in range(k))
              for n in range(N)] for t in range(T)]
    for t in range(T):
        for n in range(N):
            assert abs(Fraction(out[t, n]) - exact[t][n]) <= Fraction(gamma(k + 1, U64)) * Fraction(ab[t, n])
    # one-hot gates pick one row exactly; k = 1 with gate 1 is the identity
    sel = rng.integers(0, k, T)
    oh = np.zeros((T, k), np.float32)
    oh[np.arange(T), sel] = 1.0
    assert np.array_equal(oracle.combine_topk(y, oh), y[np.arange(T) * k + sel])
    assert np.array_equal(oracle.combine_topk(y, np.ones((T * k, 1), np.float32)), y)
    # a gate of 2 doubles its row exactly
    assert np.array_equal(oracle.combine_topk(y, 2 * oh), 2 * y[np.arange(T) * k + sel])


# ----------------------------------------------- gated activations ------

def test_silu_closed_forms_and_logistic_identity():
    from scipy.special import expit
    assert oracle.act(oracle.ACT_SILU, 0.0) == 0.0
    assert abs(oracle.act(oracle.ACT_SILU, np.log(3.0)) - 0.75 * np.log(3.0)) <= 4 * U64
    rng = np.random.default_rng(3)
    for x in np.concatenate([rng.standard_normal(200) * 4, [-30.0, -7.5, 7.5, 30.0]]):
        s, sm = oracle.act(oracle.ACT_SILU, x), oracle.act(oracle.ACT_SILU, -x)
        assert abs((s - sm) - x) <= 8 * U64 * (abs(x) + 1)            # silu(x) - silu(-x) = x
        assert abs(s - x * expit(x)) <= 8 * U64 * (abs(x) + 1)        # x * logistic(x)


def test_gelu_tanh_identities_and_distance_to_erf_gelu():
    from scipy.special import erf
    assert oracle.act(oracle.ACT_GELU_TANH, 0.0) == 0.0
    xs = np.linspace(-9.0, 9.0, 3601)
    g = np.array([oracle.act(oracle.ACT_GELU_TANH, x) for x in xs])
    gm = np.array([oracle.act(oracle.ACT_GELU_TANH, -x) for x in xs])
    assert np.all(np.abs((g - gm) - xs) <= 16 * U64 * (np.abs(xs) + 1))   # odd part is x / 2
    exact_gelu = 0.5 * xs * (1 + erf(xs / np.sqrt(2.0)))
    # the tanh form approximates the erf form to within 5e-4 everywhere; a wrong
    # constant (0.44715 for 0.044715, sqrt(2 pi) for sqrt(2 / pi)) misses by > 1e-3
    assert np.abs(g - exact_gelu).max() <= 5e-4
    assert abs(oracle.act(oracle.ACT_GELU_TANH, 9.0) - 9.0) < 1e-12       # saturates to x


def _act_grid():
    rng = np.random.default_rng(11)
    return np.concatenate([np.linspace(-9.0, 9.0, 1801), rng.standard_normal(2000) * 3, [-20.0, -0.0, 20.0]])


def test_activations_match_torch_float64_to_a_few_ulps():
    """The oracle's SiLU and tanh-form GELU against torch's own float64
    implementations (an independent code base): agreement within a few fp64
    ulps of (|x| + 1) everywhere on a grid over +-9 and random points pins
    every constant of both formulas (FreeToken PR #185, Problem: the
    gelu_tanh_and_mul after the GEMV; "Current Bug: CuTeDSLMoERunner", Bug 6:
    SiLU * up)."""
    import torch
    import torch.nn.functional as F
    xs = _act_grid()
    tol = 32 * U64 * (np.abs(xs) + 1)
    tx = torch.from_numpy(xs)
    ref_gelu = F.gelu(tx, approximate="tanh").numpy()
    ref_silu = F.silu(tx).numpy()
    g = np.array([oracle.act(oracle.ACT_GELU_TANH, x) for x in xs])
    s = np.array([oracle.act(oracle.ACT_SILU, x) for x in xs])
    assert np.all(np.abs(g - ref_gelu) <= tol)
    assert np.all(np.abs(s - ref_silu) <= tol)


def test_activation_pin_rejects_mistyped_constants():
    """The tolerance of the torch comparison is tight enough that a dropped
    digit of the cubic coefficient or a rounded sqrt(2/pi) fails it (the
    distance-to-erf check alone passes 0.0447 and 0.04471)."""
    import torch
    import torch.nn.functional as F
    xs = _act_grid()
    tol = 32 * U64 * (np.abs(xs) + 1)
    ref = F.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    k = np.sqrt(2.0 / np.pi)
    for kk, c in ((k, 0.0447), (k, 0.04471), (0.8, 0.044715), (k, 0.44715)):
        wrong = 0.5 * xs * (1.0 + np.tanh(kk * (xs + c * xs ** 3)))
        assert np.any(np.abs(wrong - ref) > tol), (kk, c)
    right = 0.5 * xs * (1.0 + np.tanh(k * (xs + 0.044715 * xs ** 3)))
    assert np.all(np.abs(right - ref) <= tol)


def test_act_and_mul_takes_gate_from_the_first_half():
    y = np.array([[np.log(3.0), -1.0, 2.0, 5.0],
                  [0.0, 2.5, 7.0, -3.0]])
    out = oracle.act_and_mul(y, oracle.ACT_SILU)
    assert out.shape == (2, 2)
    assert abs(out[0, 0] - 0.75 * np.log(3.0) * 2.0) <= 8 * U64
    assert out[1, 0] == 0.0                                            # silu(0) * 7
    s25 = oracle.act(oracle.ACT_SILU, 2.5)
    assert out[1, 1] == s25 * -3.0
    swapped = oracle.act_and_mul(np.concatenate([y[:, 2:], y[:, :2]], axis=1), oracle.ACT_SILU)
    assert not np.allclose(swapped, out)


# ------------------------------------------- sibling GGUF block types ------

SIBLINGS = [oracle.W_Q4_1, oracle.W_Q5_0, oracle.W_Q5_1, oracle.W_Q8_0]


def _tiny_w(wtype, seed=0, E=3, top_k=2, T=3, K=96, N=5):
    w = oracle.quantize_w(wtype, inputs.weights(E, N, K, seed=seed) * 40)   # spread codes over the range
    a = oracle.quantize_q8_1(inputs.activations(T, K, seed=seed))
    ids = inputs.routing(T, E, top_k, seed=seed)
    return w, a, ids, dict(E=E, N=N, K=K, T=T, top_k=top_k)


@pytest.mark.parametrize("wtype", SIBLINGS)
def test_sibling_exact_rational_bruteforce(wtype):
    """Independent numpy decode, exact Fractions; fp64 error within gamma(2 nb) * sum of |parts|."""
    w, a, ids, c = _tiny_w(wtype, seed=wtype)
    out, ab = oracle.moe_w(wtype, w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"], want_abssum=True)
    d, m, q, z = _decode.gguf_w(wtype, w.reshape(c["E"], c["N"], -1), c["K"])
    ad, _, aq = _decode.q8_1(a, c["K"])
    nb = c["K"] // 32
    for p in range(c["T"] * c["top_k"]):
        t, e = p // c["top_k"], int(ids.reshape(-1)[p])
        for n in range(c["N"]):
            exact = Fraction(0)
            for b in range(nb):
                P = sum((int(q[e, n, b, i]) - z) * int(aq[t, b, i]) for i in range(32))
                S = sum(int(aq[t, b, i]) for i in range(32))
                exact += Fraction(ad[t, b]) * (Fraction(d[e, n, b]) * P + Fraction(m[e, n, b]) * S)
            assert abs(Fraction(out[p, n]) - exact) <= Fraction(gamma(2 * nb, U64)) * Fraction(ab[p, n])


@pytest.mark.parametrize("wtype", SIBLINGS)
def test_sibling_partials_match_integer_einsum(wtype):
    w, a, ids, c = _tiny_w(wtype, seed=1, E=4, T=9, K=256, N=17)
    P = oracle.moe_w_partials(wtype, w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"])
    _, _, q, z = _decode.gguf_w(wtype, w.reshape(c["E"], c["N"], -1), c["K"])
    _, _, aq = _decode.q8_1(a, c["K"])
    tok = np.arange(c["T"] * c["top_k"]) // c["top_k"]
    ref = np.einsum("pnbi,pbi->pnb", q[ids.reshape(-1)] - z, aq[tok])
    assert P.dtype == np.int32 and np.array_equal(P, ref)


def test_generic_path_reproduces_q4_0():
    w, a, ids, c = _tiny(seed=9)
    assert np.array_equal(oracle.moe_w(oracle.W_Q4_0, w, a, ids, c["E"], c["N"], c["K"], c["T"], c["top_k"]),
                          _run(w, a, ids, c))


@pytest.mark.parametrize("wtype", SIBLINGS)
def test_sibling_quantizers_recover_exact_grids(wtype):
    rng = np.random.default_rng(wtype)
    levels = {oracle.W_Q4_1: 15, oracle.W_Q5_0: 31, oracle.W_Q5_1: 31, oracle.W_Q8_0: 254}[wtype]
    d = 2.0 ** -6
    rows = []
    for _ in range(16):
        q = rng.integers(0, levels + 1, 32)
        q[0], q[1] = 0, levels                       # both ends present: the range is levels * d
        if wtype == oracle.W_Q5_0:
            q[1] = 0; q[2] = 31 - 15                 # extreme -16 * d: (0 - 16) d sets d
            rows.append((q - 16) * d)
        elif wtype == oracle.W_Q8_0:
            rows.append((q - 127) * d)               # |x| <= 127 d with 127 d present
        else:
            rows.append(q * d - 0.5)                 # offset -0.5: m = min = -0.5
    x = np.array(rows, np.float32)
    y = oracle.quantize_w(wtype, x)
    dd, mm, qq, z = _decode.gguf_w(wtype, y, 32)
    back = dd[..., None] * (qq - z) + mm[..., None]
    assert np.array_equal(back.reshape(x.shape).astype(np.float32), x)


def test_sibling_layout_closed_forms():
    a = np.zeros((1, 36), np.uint8)                  # one Q8_1 block: d8 = 0.5, codes 1..32 at element i
    a[0, 0:2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    a[0, 4:36] = np.arange(1, 33, dtype=np.int8).view(np.uint8)
    ids = np.zeros((1, 1), np.int32)
    S = sum(range(1, 33))
    # Q4_1 with every nibble 0: every weight is m, so out = m * d8 * S
    w = np.zeros(20, np.uint8)
    w[0:2] = np.frombuffer(np.float16(0.25).tobytes(), np.uint8)
    w[2:4] = np.frombuffer(np.float16(-1.5).tobytes(), np.uint8)
    assert oracle.moe_w(oracle.W_Q4_1, w, a.reshape(-1), ids, 1, 1, 32, 1, 1)[0, 0] == -1.5 * 0.5 * S
    # Q5_0: qh bit 21 and nibble 15 of element 21 (high nibble of byte 5) give q = 31, others q = 16 (zero)
    w = np.zeros(22, np.uint8)
    w[0:2] = np.frombuffer(np.float16(0.125).tobytes(), np.uint8)
    w[2:6] = np.frombuffer(np.uint32(1 << 21).tobytes(), np.uint8)
    w[6:22] = 0x00
    w[6 + 5] = 0xF0
    qh_other = np.uint32(0xFFFFFFFF ^ (1 << 21))     # every other element: bit 4 set, nibble 0 -> 16
    w[2:6] = np.frombuffer(np.uint32(qh_other | (1 << 21)).tobytes(), np.uint8)
    assert oracle.moe_w(oracle.W_Q5_0, w, a.reshape(-1), ids, 1, 1, 32, 1, 1)[0, 0] == 15 * 0.125 * 0.5 * 22
    # Q8_0: code -3 at element 7 only
    w = np.zeros(34, np.uint8)
    w[0:2] = np.frombuffer(np.float16(2.0).tobytes(), np.uint8)
    w[2 + 7] = np.uint8(np.int8(-3).view(np.uint8))
    assert oracle.moe_w(oracle.W_Q8_0, w, a.reshape(-1), ids, 1, 1, 32, 1, 1)[0, 0] == -3 * 2.0 * 0.5 * 8
