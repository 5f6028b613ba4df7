"""The grouped path's three kernels against the oracle and against each other.

The grouped path computes each 32-block's integer partial exactly, either on
int8 MFMAs (the default), on two fp16 MFMAs, or on fp16 MFMAs in a
warp-specialised kernel (128-row tiles), then scales it with one fp32 FMA per
element and block in ascending block order.  The choice changes nothing but
speed: each kernel must give the oracle's integer partials bit for bit (the
exact block dot of the FreeToken PR #185 Q4_0 x Q8_1 GEMV, "Problem"), and the
three must give the same fp32 output bits, on the plain, per-pair, fused-gated
and partials entry points, with ragged tiles, empty experts and skewed routing.
"""
import numpy as np
import pytest
import torch

from quantized_moe_expert_quantize_amd import ftq
from tests._cases import Case, assert_matches_oracle, sample_pairs, say
from tests.test_gpu_down import PairCase

pytestmark = pytest.mark.gpu

VARIANTS = (ftq.GROUPED_I8, ftq.GROUPED_F16, ftq.GROUPED_F16_WS)


@pytest.fixture(autouse=True)
def _default_kernel_after():
    yield
    ftq.grouped_kernel(ftq.GROUPED_I8)


def _each_variant(fn):
    outs = []
    for v in VARIANTS:
        ftq.grouped_kernel(v)
        r = fn()
        torch.cuda.synchronize()
        outs.append(r)
    ftq.grouped_kernel(ftq.GROUPED_I8)
    return outs


# (E, N, K, T, top_k, routing): >= 96 pairs per expert on average selects 128-row
# tiles, where all three kernels run; N and the per-expert counts leave ragged tiles
SHAPES = [
    (4, 200, 320, 100, 4, "uniform"),
    (8, 136, 512, 400, 2, "zipf"),
    (6, 64, 96, 150, 4, "uniform"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "E{}N{}K{}T{}k{}{}".format(*s))
def test_kernels_partials_exact_and_outputs_identical(shape):
    E, N, K, T, k, kind = shape
    say(f"[grouped kernels] {shape}")
    c = Case(E, N, K, T, k, seed=11, kind=kind)
    ref_part = c.oracle_partials()
    parts = _each_variant(lambda: c.partials(ftq.PATH_GROUPED))
    for v, p in zip(VARIANTS, parts):
        assert np.array_equal(p, ref_part), f"variant {v}: partials differ from the oracle"
    outs = _each_variant(lambda: c.run(ftq.PATH_GROUPED).clone())
    for v, o in zip(VARIANTS[1:], outs[1:]):
        assert torch.equal(o, outs[0]), f"variant {v}: output bits differ from the int8 kernel"
    ref, ab = c.oracle_out()
    assert_matches_oracle(outs[0].cpu().numpy(), ref, ab, c.nb)


def test_kernels_per_pair_rows():
    E, N, K, T, k = 4, 160, 256, 110, 4
    c = PairCase(E, N, K, T, k, seed=12)
    parts = _each_variant(lambda: c.partials(ftq.PATH_GROUPED))
    ref_part = c.oracle_partials()
    for v, p in zip(VARIANTS, parts):
        assert np.array_equal(p, ref_part), f"variant {v}"
    outs = _each_variant(lambda: c.run(ftq.PATH_GROUPED).clone())
    for v, o in zip(VARIANTS[1:], outs[1:]):
        assert torch.equal(o, outs[0]), f"variant {v}"
    ref, ab = c.oracle_out()
    assert_matches_oracle(outs[0].cpu().numpy(), ref, ab, c.nb)


@pytest.mark.parametrize("act", [ftq.ACT_SILU, ftq.ACT_GELU_TANH])
def test_kernels_fused_gated_activation(act):
    E, N, K, T, k = 4, 2 * 72, 256, 200, 2
    c = Case(E, N, K, T, k, seed=13)
    wq, aq, ids = c.gpu()
    outs = _each_variant(lambda: ftq.moe_act(wq, aq, ids, E, N, K, act, path=ftq.PATH_GROUPED).clone())
    for v, o in zip(VARIANTS[1:], outs[1:]):
        assert torch.equal(o, outs[0]), f"variant {v}"
    # the epilogue pairs gate column n with up column n + N/2 of the plain product
    plain = c.run(ftq.PATH_GROUPED).double()
    g, u = plain[:, : N // 2], plain[:, N // 2:]
    ref = (g * torch.sigmoid(g) if act == ftq.ACT_SILU else
           0.5 * g * (1 + torch.tanh(0.7978845608028654 * (g + 0.044715 * g ** 3)))) * u
    got = outs[0].double()
    assert torch.allclose(got, ref, rtol=1e-5, atol=1e-6 * float(ref.abs().max()))


def test_kernels_page1_shape_sampled():
    # the page-1 expert shape (E = 128, N = 1408, K = 2816, top_k = 8) at T = 2048:
    # all three kernels bit-equal over the whole output, sampled pairs against the oracle
    E, N, K, T, k = 128, 1408, 2816, 2048, 8
    c = Case(E, N, K, T, k, seed=0)
    outs = _each_variant(lambda: c.run(ftq.PATH_GROUPED).clone())
    for v, o in zip(VARIANTS[1:], outs[1:]):
        assert torch.equal(o, outs[0]), f"variant {v}"
    pairs = sample_pairs(T, k, 24, seed=3)
    ref, ab = c.oracle_out(pairs)
    assert_matches_oracle(outs[0].cpu().numpy()[pairs], ref, ab, c.nb)


def test_kernels_partials_exact_at_page1_K_with_128_row_tiles():
    # the page-1 hidden size (K = 2816, 88 blocks: 44 passes) at the tile height
    # the bench runs (>= 96 pairs per expert), on a reduced N
    E, N, K, T, k = 4, 160, 2816, 120, 4
    c = Case(E, N, K, T, k, seed=14)
    ref_part = c.oracle_partials()
    parts = _each_variant(lambda: c.partials(ftq.PATH_GROUPED))
    for v, p in zip(VARIANTS, parts):
        assert np.array_equal(p, ref_part), f"variant {v}"
    ref, ab = c.oracle_out()
    assert_matches_oracle(c.run(ftq.PATH_GROUPED).cpu().numpy(), ref, ab, c.nb)


def test_unknown_variant_is_rejected():
    with pytest.raises(RuntimeError, match="variant"):
        ftq.grouped_kernel(7)
