"""Independent numpy decoders of the Q4_0 / Q8_1 block bytes, used by tests to
build brute-force references (numpy's own float16 conversion, vectorised bit
operations) that share nothing with the oracle's C code."""
import numpy as np


def q4_0(w_bytes: np.ndarray, K: int):
    """uint8 [..., K/32*18] -> (d float64 [..., K/32], q int64 [..., K/32, 32] in [-8, 7])."""
    nb = K // 32
    lead = w_bytes.shape[:-1]
    blk = np.ascontiguousarray(w_bytes).reshape(lead + (nb, 18))
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    qs = blk[..., 2:18].astype(np.int64)
    q = np.concatenate([qs & 15, qs >> 4], axis=-1) - 8
    return d, q


def q8_1(a_bytes: np.ndarray, K: int):
    """uint8 [..., K/32*36] -> (d float64, s float64 [..., K/32], q int64 [..., K/32, 32])."""
    nb = K // 32
    lead = a_bytes.shape[:-1]
    blk = np.ascontiguousarray(a_bytes).reshape(lead + (nb, 36))
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    s = blk[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    q = blk[..., 4:36].copy().view(np.int8).astype(np.int64)
    return d, s, q
