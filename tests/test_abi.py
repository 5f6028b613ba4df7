"""The C ABI on the host: the library loads, exports every function that
include/ftq.h declares, and rejects bad arguments before anything reaches the
GPU (no call here touches a device)."""
import ctypes
import os
import re

import pytest

from quantized_moe_expert_quantize_amd import ftq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "ftq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ftq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(ftq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ftq.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version():
    assert ftq.version().startswith("ftq ") and "gfx950" in ftq.version()


def _moe(L, w=1, a=1, ids=1, out=1, E=8, N=64, K=256, T=4, k=2, ws=None, wsb=0, path=0):
    P = lambda v: ctypes.c_void_p(v) if v else None
    return L.ftq_moe_q4_0_q8_1(P(w and 0x1000 * w), P(a and 0x2000 * a), P(ids and 0x3000 * ids),
                               P(out and 0x4000 * out), E, N, K, T, k, P(ws), wsb, path, None)


@pytest.mark.parametrize("kw", [
    dict(K=250), dict(K=0), dict(K=-32), dict(E=0), dict(N=0), dict(k=0), dict(T=-1),
    dict(k=9), dict(path=7), dict(w=0), dict(a=0), dict(ids=0), dict(out=0),
])
def test_moe_rejects_invalid_arguments(kw):
    L = ftq.lib()
    assert _moe(L, **kw) == ftq.ERR_INVALID_ARG
    assert ftq.last_error()


def test_moe_rejects_misaligned_pointers():
    L = ftq.lib()
    P = ctypes.c_void_p
    base = 0x100000
    args = [P(base), P(base), P(base), P(base)]
    for i, off in ((0, 1), (1, 2), (2, 2), (3, 2)):
        bad = list(args)
        bad[i] = P(base + off)
        assert L.ftq_moe_q4_0_q8_1(*bad, 8, 64, 256, 4, 2, None, 0, ftq.PATH_GEMV, None) == ftq.ERR_INVALID_ARG
        assert "misaligned" in ftq.last_error()


def test_moe_limits_are_unsupported_not_overflowing():
    L = ftq.lib()
    assert _moe(L, T=2 ** 31, k=1, E=1) == ftq.ERR_UNSUPPORTED
    assert "2^31" in ftq.last_error()
    assert _moe(L, E=5000, k=2) == ftq.ERR_UNSUPPORTED


def test_moe_zero_tokens_is_a_noop():
    L = ftq.lib()
    assert _moe(L, T=0, w=0, a=0, ids=0, out=0) == ftq.OK
    assert ftq.workspace_bytes(8, 64, 256, 0, 2) == 0


def test_grouped_needs_workspace():
    L = ftq.lib()
    need = ftq.workspace_bytes(8, 64, 256, 64, 2, ftq.PATH_GROUPED)
    assert need > 0
    assert _moe(L, T=64, path=ftq.PATH_GROUPED) == ftq.ERR_WORKSPACE
    assert _moe(L, T=64, path=ftq.PATH_GROUPED, ws=0x100000, wsb=need - 1) == ftq.ERR_WORKSPACE
    assert _moe(L, T=64, path=ftq.PATH_GROUPED, ws=0x100010, wsb=need) == ftq.ERR_INVALID_ARG  # not 256-aligned


def test_path_choice_is_host_arithmetic_of_sizes():
    # decode sizes take the GEMV path, prefill sizes the grouped MFMA path
    assert ftq.select_path(8, 14336, 4096, 1, 2) == ftq.PATH_GEMV
    assert ftq.select_path(8, 14336, 4096, 8, 2) == ftq.PATH_GEMV
    assert ftq.select_path(8, 14336, 4096, 64, 2) == ftq.PATH_GROUPED
    assert ftq.select_path(128, 1408, 2816, 1, 8) == ftq.PATH_GEMV
    # measured crossovers: ~7 pairs per expert at 8 experts, ~4 at 128
    assert ftq.select_path(8, 14336, 4096, 28, 2) == ftq.PATH_GEMV      # 7 per expert
    assert ftq.select_path(8, 14336, 4096, 32, 2) == ftq.PATH_GROUPED   # 8 per expert
    assert ftq.select_path(128, 1408, 2816, 64, 8) == ftq.PATH_GEMV     # 4 per expert
    assert ftq.select_path(128, 1408, 2816, 65, 8) == ftq.PATH_GROUPED  # just over 4 per expert
    for T in (2048, 4096, 8191, 8192, 16384):
        assert ftq.select_path(128, 1408, 2816, T, 8) == ftq.PATH_GROUPED
    assert ftq.workspace_bytes(8, 14336, 4096, 1, 2) == 0
    with pytest.raises(ftq.FtqError):
        ftq.select_path(8, 14336, 4095, 1, 2)


def test_workspace_is_monotone_and_exact_for_bucketing():
    prev = 0
    for T in (64, 1000, 4096, 8192, 16384):
        b = ftq.workspace_bytes(128, 1408, 2816, T, 8, ftq.PATH_GROUPED)
        assert b >= 4 * T * 8 and b > prev
        prev = b


def test_quantize_rejects_invalid_arguments():
    L = ftq.lib()
    P = ctypes.c_void_p
    assert L.ftq_quantize_q8_1(P(0x1000), 4, 48, P(0x2000), None) == ftq.ERR_INVALID_ARG
    assert L.ftq_quantize_q8_1(P(0x1004), 4, 64, P(0x2000), None) == ftq.ERR_INVALID_ARG
    assert L.ftq_quantize_q8_1(None, 4, 64, P(0x2000), None) == ftq.ERR_INVALID_ARG
    assert L.ftq_quantize_q8_1(None, 0, 64, None, None) == ftq.OK
    assert L.ftq_quantize_q4_0(P(0x1000), 4, 40, P(0x2000), None) == ftq.ERR_INVALID_ARG
    assert L.ftq_quantize_q4_0(P(0x1000), 4, 64, P(0x2001), None) == ftq.ERR_INVALID_ARG
    assert L.ftq_quantize_q4_0(None, 0, 64, None, None) == ftq.OK


def test_pairs_and_combine_validate_before_any_launch():
    """Argument checks of the second-layer calls run on the host and never reach a kernel."""
    L = ftq.lib()
    P = ctypes.c_void_p
    base = P(0x100000)
    # per-pair matmul: the same size and pointer rules as the per-token call
    assert L.ftq_moe_q4_0_q8_1_pairs(base, base, base, base, 8, 64, 250, 4, 2, None, 0, ftq.PATH_GEMV, None) == ftq.ERR_INVALID_ARG
    assert L.ftq_moe_q4_0_q8_1_pairs(base, None, base, base, 8, 64, 256, 4, 2, None, 0, ftq.PATH_GEMV, None) == ftq.ERR_INVALID_ARG
    assert L.ftq_moe_q4_0_q8_1_pairs(None, None, None, None, 8, 64, 256, 0, 2, None, 0, ftq.PATH_AUTO, None) == ftq.OK
    assert L.ftq_moe_q4_0_q8_1_pairs_partials(base, base, base, None, 8, 64, 256, 4, 2, None, 0, ftq.PATH_GEMV, None) == ftq.ERR_INVALID_ARG
    # the workspace holds the bucket tables only (both paths read the Q8_1 rows
    # in place), so per-pair rows need no more of it than per-token rows
    E, N, K, T, k = 128, 1408, 2816, 8191, 8
    tok = ftq.workspace_bytes(E, N, K, T, k, ftq.PATH_GROUPED)
    pp = ftq.pairs_workspace_bytes(E, N, K, T, k, ftq.PATH_GROUPED)
    assert pp == tok > 0
    assert tok < 8 * T * k   # sorted pair ids, per-chunk counts and per-bucket tables: a few int32 per pair
    assert ftq.pairs_workspace_bytes(E, N, K, T, k, ftq.PATH_GEMV) == ftq.workspace_bytes(E, N, K, T, k, ftq.PATH_GEMV)
    assert L.ftq_moe_q4_0_q8_1_pairs(base, base, base, base, E, N, K, T, k, base, tok - 1, ftq.PATH_GROUPED, None) == ftq.ERR_WORKSPACE
    assert "workspace" in ftq.last_error()
    # combine
    assert L.ftq_moe_combine_topk(None, None, None, 0, 2, 16, None) == ftq.OK
    assert L.ftq_moe_combine_topk(base, base, None, 3, 2, 16, None) == ftq.ERR_INVALID_ARG
    assert L.ftq_moe_combine_topk(base, P(0x100002), base, 3, 2, 16, None) == ftq.ERR_INVALID_ARG
    assert "misaligned" in ftq.last_error()
    for T_, k_, N_ in ((-1, 2, 16), (3, 0, 16), (3, 2, 0)):
        assert L.ftq_moe_combine_topk(base, base, base, T_, k_, N_, None) == ftq.ERR_INVALID_ARG
    assert L.ftq_moe_combine_topk(base, base, base, 2 ** 40, 8, 2 ** 20, None) == ftq.ERR_UNSUPPORTED


# Mixtral down projection (mlxcel PR #652, Summary: mixtral-8x7b; the second
# layer's K is the expert width 14336): at T = 12 and 16 an expert holds 3-4
# pairs and their staged rows exceed the LDS budget, so the GEMV streams each
# row in K segments.  The GPU tests of those shapes rely on this plan.
KSEG_SHAPES = [(8, 4096, 14336, 12, 2), (8, 4096, 14336, 16, 2), (8, 96, 14336, 16, 2), (4, 48, 20480, 8, 2)]


@pytest.mark.parametrize("shape", KSEG_SHAPES)
def test_gemv_plan_streams_long_rows_in_segments(shape):
    E, N, K, T, k = shape
    plan = ftq.gemv_plan(E, N, K, T, k)
    nb = K // 32
    assert plan["seg"] < nb and plan["seg"] % 128 == 0, plan
    assert plan["pairs_per_pass"] >= 3


def test_gemv_plan_one_segment_for_decode_rows():
    # the halves of the T = 16 batch (T = 8) stage whole rows: one segment
    assert ftq.gemv_plan(8, 4096, 14336, 8, 2)["seg"] == 14336 // 32
    assert ftq.gemv_plan(8, 14336, 4096, 1, 2)["seg"] == 4096 // 32
    assert ftq.gemv_plan(128, 1408, 2816, 16, 8)["seg"] == 2816 // 32
    # a fused activation needs whole rows: one segment or an error
    assert ftq.gemv_plan(8, 28672, 4096, 8, 2, act=1)["seg"] == 4096 // 32
    with pytest.raises(ftq.FtqError):
        ftq.gemv_plan(8, 64, 33056 + 32, 1, 2, act=1)
