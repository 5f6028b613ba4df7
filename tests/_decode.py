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


def gguf_w(wtype: int, w_bytes: np.ndarray, K: int):
    """Sibling GGUF block types -> (d, m float64 [..., nb], codes int64 [..., nb, 32], zero point).
    Byte layouts: Q4_1 (3) d, m, 16 nibble bytes; Q5_0 (6) d, qh (uint32 LE), nibbles;
    Q5_1 (7) d, m, qh, nibbles; Q8_0 (8) d, 32 int8; Q4_0 (2) d, nibbles."""
    nb = K // 32
    size = {2: 18, 3: 20, 6: 22, 7: 24, 8: 34}[wtype]
    lead = w_bytes.shape[:-1]
    blk = np.ascontiguousarray(w_bytes).reshape(lead + (nb, size))
    f16 = lambda o: blk[..., o:o + 2].copy().view(np.float16)[..., 0].astype(np.float64)
    d = f16(0)
    m = np.zeros_like(d)
    if wtype == 8:
        return d, m, blk[..., 2:34].copy().view(np.int8).astype(np.int64), 0
    if wtype in (3, 7):
        m = f16(2)
    off = {2: 2, 3: 4, 6: 6, 7: 8}[wtype]
    qs = blk[..., off:off + 16].astype(np.int64)
    q = np.concatenate([qs & 15, qs >> 4], axis=-1)
    if wtype in (6, 7):
        ho = 2 if wtype == 6 else 4
        qh = blk[..., ho:ho + 4].copy().view(np.uint32)[..., 0].astype(np.int64)
        bits = (qh[..., None] >> np.arange(32)) & 1
        q = q | (bits << 4)
    zero = {2: 8, 3: 0, 6: 16, 7: 0}[wtype]
    return d, m, q, zero
