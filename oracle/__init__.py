"""CPU oracle for the Q4_0 x Q8_1 mixture-of-experts expert matmul.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product library never does.
It shares no code with the HIP library.  ``oracle.c`` holds the arithmetic;
this module only builds it with gcc and marshals numpy arrays through ctypes.

Every function follows the definition spelled out at the top of ``oracle.c``:
per (token, top-k) pair, the routed expert's Q4_0 rows dotted block by block
with the token's Q8_1 row [FreeToken PR #185, "fix(kernel): launch GGUF MoE
GEMV token axis on grid.x, not grid.z", sections Problem and Fix].  With
``per_pair=True`` each pair reads its own activation row instead (the second
layer of an expert FFN, whose input is the first layer's per-pair output
["Current Bug: CuTeDSLMoERunner", Bug 6]); ``combine_topk`` is the per-token
router-weighted sum of the pair outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB_PATH: a build of oracle.c made elsewhere (the host-sanitizer run)
_LIB_ENV = os.environ.get("ORACLE_LIB_PATH")
_LIB = _LIB_ENV or os.path.join(_HERE, "liboracle.so")
QK = 32
Q4_0_BYTES = 18
Q8_1_BYTES = 36

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain C, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_ENV and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_fp16_to_fp32.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_fp32.restype = ctypes.c_float
    lib.oracle_fp32_to_fp16.argtypes = [ctypes.c_float]
    lib.oracle_fp32_to_fp16.restype = ctypes.c_uint16
    lib.oracle_fp16_to_fp32_array.argtypes = [P, I64, P]
    lib.oracle_fp32_to_fp16_array.argtypes = [P, I64, P]
    lib.oracle_quantize_q8_1.argtypes = [P, I64, I64, P]
    lib.oracle_quantize_q4_0.argtypes = [P, I64, I64, P]
    lib.oracle_moe.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, P]
    lib.oracle_moe_pairs.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, I64, P, P]
    lib.oracle_moe_partials.argtypes = [P, P, P, I64, I64, I64, I64, I64, P]
    lib.oracle_moe_ex.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P, P]
    lib.oracle_moe_pairs_ex.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P, I64, P, P]
    lib.oracle_moe_partials_ex.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P]
    lib.oracle_combine_topk.argtypes = [P, P, I64, I64, I64, P, P]
    I32 = ctypes.c_int
    lib.oracle_w_block_bytes.argtypes = [I32]
    lib.oracle_w_block_bytes.restype = I32
    lib.oracle_quantize_w.argtypes = [I32, P, I64, I64, P]
    lib.oracle_moe_w_pairs.argtypes = [I32, P, P, P, I64, I64, I64, I64, P, I64, P, P]
    lib.oracle_moe_w_partials.argtypes = [I32, P, P, P, I64, I64, I64, I64, I64, I64, P]
    lib.oracle_act.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_act.restype = ctypes.c_double
    lib.oracle_act_and_mul.argtypes = [P, I64, I64, ctypes.c_int, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def fp16_to_fp32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    f = np.empty(h.shape, np.float32)
    _load().oracle_fp16_to_fp32_array(_ptr(h), h.size, _ptr(f))
    return f


def fp32_to_fp16(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    h = np.empty(f.shape, np.uint16)
    _load().oracle_fp32_to_fp16_array(_ptr(f), f.size, _ptr(h))
    return h


def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """fp32 [rows, K] -> uint8 [rows, K/32*36] (Q8_1 blocks)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    assert K % QK == 0
    y = np.empty((rows, K // QK * Q8_1_BYTES), np.uint8)
    _load().oracle_quantize_q8_1(_ptr(x), rows, K, _ptr(y))
    return y


def quantize_q4_0(w: np.ndarray) -> np.ndarray:
    """fp32 [..., K] -> uint8 [..., K/32*18] (Q4_0 blocks), leading dims kept."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    assert K % QK == 0
    rows = w.size // K
    y = np.empty(w.shape[:-1] + (K // QK * Q4_0_BYTES,), np.uint8)
    _load().oracle_quantize_q4_0(_ptr(w), rows, K, _ptr(y))
    return y


def _check(w, a, ids, E, N, K, T, top_k, per_pair=False):
    nb = K // QK
    rows = T * top_k if per_pair else T
    assert w.dtype == np.uint8 and w.size == E * N * nb * Q4_0_BYTES and w.flags.c_contiguous
    assert a.dtype == np.uint8 and a.size == rows * nb * Q8_1_BYTES and a.flags.c_contiguous
    assert ids.dtype == np.int32 and ids.size == T * top_k and ids.flags.c_contiguous
    return 1 if per_pair else top_k


def moe(w, a, ids, E, N, K, T, top_k, want_abssum=False, per_pair=False):
    """fp64 outputs [T*top_k, N] (and sum of |block terms| if asked).

    a holds one Q8_1 row per token ([T, K/32] blocks), or one per pair
    ([T*top_k, K/32]) when per_pair is set."""
    div = _check(w, a, ids, E, N, K, T, top_k, per_pair)
    out = np.empty((T * top_k, N), np.float64)
    ab = np.empty_like(out) if want_abssum else None
    _load().oracle_moe_ex(_ptr(w), _ptr(a), _ptr(ids), E, N, K, T, top_k, div, _ptr(out),
                          _ptr(ab) if ab is not None else None)
    return (out, ab) if want_abssum else out


def moe_pairs(w, a, ids, E, N, K, T, top_k, pairs, want_abssum=False, per_pair=False):
    """fp64 outputs for the listed flat pair indices only: [len(pairs), N]."""
    div = _check(w, a, ids, E, N, K, T, top_k, per_pair)
    pairs = np.ascontiguousarray(pairs, dtype=np.int64)
    assert pairs.size == 0 or (pairs.min() >= 0 and pairs.max() < T * top_k)
    out = np.empty((pairs.size, N), np.float64)
    ab = np.empty_like(out) if want_abssum else None
    _load().oracle_moe_pairs_ex(_ptr(w), _ptr(a), _ptr(ids), E, N, K, T, top_k, div, _ptr(pairs),
                                pairs.size, _ptr(out), _ptr(ab) if ab is not None else None)
    return (out, ab) if want_abssum else out


def moe_partials(w, a, ids, E, N, K, T, top_k, per_pair=False):
    """Exact integer block partials [T*top_k, N, K/32] (int32)."""
    div = _check(w, a, ids, E, N, K, T, top_k, per_pair)
    out = np.empty((T * top_k, N, K // QK), np.int32)
    _load().oracle_moe_partials_ex(_ptr(w), _ptr(a), _ptr(ids), E, N, K, T, top_k, div, _ptr(out))
    return out


ACT_SILU, ACT_GELU_TANH = 1, 2

# GGUF block types (type ids as in GGUF files): Q4_0, Q4_1, Q5_0, Q5_1, Q8_0
W_Q4_0, W_Q4_1, W_Q5_0, W_Q5_1, W_Q8_0 = 2, 3, 6, 7, 8
W_TYPES = (W_Q4_0, W_Q4_1, W_Q5_0, W_Q5_1, W_Q8_0)


def w_block_bytes(wtype: int) -> int:
    return int(_load().oracle_w_block_bytes(int(wtype)))


def quantize_w(wtype: int, w: np.ndarray) -> np.ndarray:
    """fp32 [..., K] -> uint8 [..., K/32 * block bytes] blocks of `wtype`."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = w.shape[-1]
    assert K % QK == 0
    bb = w_block_bytes(wtype)
    rows = w.size // K
    y = np.empty(w.shape[:-1] + (K // QK * bb,), np.uint8)
    _load().oracle_quantize_w(int(wtype), _ptr(w), rows, K, _ptr(y))
    return y


def _check_w(wtype, w, a, ids, E, N, K, T, top_k, per_pair):
    nb = K // QK
    rows = T * top_k if per_pair else T
    assert w.dtype == np.uint8 and w.size == E * N * nb * w_block_bytes(wtype) and w.flags.c_contiguous
    assert a.dtype == np.uint8 and a.size == rows * nb * Q8_1_BYTES and a.flags.c_contiguous
    assert ids.dtype == np.int32 and ids.size == T * top_k and ids.flags.c_contiguous
    return 1 if per_pair else top_k


def moe_w(wtype, w, a, ids, E, N, K, T, top_k, pairs=None, want_abssum=False, per_pair=False):
    """fp64 outputs for weights of `wtype`: [T*top_k, N], or the listed pairs' rows.
    abssum holds, per element, the sum over blocks of |d d8 P| + |m d8 S|."""
    div = _check_w(wtype, w, a, ids, E, N, K, T, top_k, per_pair)
    pairs = np.arange(T * top_k, dtype=np.int64) if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64)
    out = np.empty((pairs.size, N), np.float64)
    ab = np.empty_like(out) if want_abssum else None
    _load().oracle_moe_w_pairs(int(wtype), _ptr(w), _ptr(a), _ptr(ids), E, N, K, div, _ptr(pairs), pairs.size,
                               _ptr(out), _ptr(ab) if ab is not None else None)
    return (out, ab) if want_abssum else out


def moe_w_partials(wtype, w, a, ids, E, N, K, T, top_k, per_pair=False):
    """Exact integer parts sum((q - z) * q8) [T*top_k, N, K/32] for weights of `wtype`."""
    div = _check_w(wtype, w, a, ids, E, N, K, T, top_k, per_pair)
    out = np.empty((T * top_k, N, K // QK), np.int32)
    _load().oracle_moe_w_partials(int(wtype), _ptr(w), _ptr(a), _ptr(ids), E, N, K, T, top_k, div, _ptr(out))
    return out


def act(kind: int, x: float) -> float:
    """SiLU (kind 1) or tanh-approximated GELU (kind 2) of one value, fp64."""
    return float(_load().oracle_act(int(kind), float(x)))


def act_and_mul(y, kind: int):
    """fp64 [rows, I]: act(y[:, :I]) * y[:, I:] for y [rows, 2I] (gate half first)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    assert y.ndim == 2 and y.shape[1] % 2 == 0
    rows, I = y.shape[0], y.shape[1] // 2
    out = np.empty((rows, I), np.float64)
    _load().oracle_act_and_mul(_ptr(y), rows, I, int(kind), _ptr(out))
    return out


def combine_topk(y, gates, want_abssum=False):
    """fp64 [T, N]: out[t] = sum_j gates[t, j] * y[t*top_k + j] (and sum of |terms|).

    y: float [T*top_k, N] (taken as fp64); gates: float32 [T, top_k]."""
    gates = np.ascontiguousarray(gates, dtype=np.float32)
    T, top_k = gates.shape
    y = np.ascontiguousarray(y, dtype=np.float64)
    assert y.ndim == 2 and y.shape[0] == T * top_k
    N = y.shape[1]
    out = np.empty((T, N), np.float64)
    ab = np.empty_like(out) if want_abssum else None
    _load().oracle_combine_topk(_ptr(y), _ptr(gates), T, top_k, N, _ptr(out),
                                _ptr(ab) if ab is not None else None)
    return (out, ab) if want_abssum else out
