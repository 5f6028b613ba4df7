"""Thin Python binding of libftq (the C ABI declared in include/ftq.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libftq.so.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or the device is not a GPU,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# FTQ_LIB_PATH: a libftq.so built elsewhere (for example with host sanitizers)
LIB_PATH = os.environ.get("FTQ_LIB_PATH") or os.path.join(_PKG, "libftq.so")

OK, ERR_INVALID_ARG, ERR_WORKSPACE, ERR_LAUNCH, ERR_UNSUPPORTED, ERR_HIP = range(6)
PATH_AUTO, PATH_GEMV, PATH_GROUPED = 0, 1, 2
ACT_SILU, ACT_GELU_TANH = 1, 2
# grouped-path kernels (same bits, different speed); GROUPED_I8 is the default
GROUPED_I8, GROUPED_F16, GROUPED_F16_WS = 0, 1, 2
# weight block types (GGUF type ids) and their block bytes
W_Q4_0, W_Q4_1, W_Q5_0, W_Q5_1, W_Q8_0 = 2, 3, 6, 7, 8
W_BLOCK_BYTES = {W_Q4_0: 18, W_Q4_1: 20, W_Q5_0: 22, W_Q5_1: 24, W_Q8_0: 34}
GEMV_ONLY = (W_Q5_0, W_Q5_1)   # the other types also run on the grouped path
QK, Q4_0_BYTES, Q8_1_BYTES = 32, 18, 36

EXPORTS = (
    "ftq_quantize_q8_1", "ftq_quantize_q4_0", "ftq_moe_select_path", "ftq_moe_workspace_bytes",
    "ftq_moe_q4_0_q8_1", "ftq_moe_route", "ftq_moe_q4_0_q8_1_routed", "ftq_moe_q4_0_q8_1_partials",
    "ftq_moe_pairs_workspace_bytes", "ftq_moe_q4_0_q8_1_pairs", "ftq_moe_q4_0_q8_1_pairs_routed",
    "ftq_moe_q4_0_q8_1_pairs_partials", "ftq_moe_combine_topk",
    "ftq_moe_q4_0_q8_1_act", "ftq_moe_q4_0_q8_1_act_routed",
    "ftq_moe_gguf_q8_1", "ftq_moe_gguf_q8_1_partials",
    "ftq_last_error", "ftq_version",
    "ftq_debug_force_block_threads", "ftq_debug_grouped_kernel", "ftq_debug_route_kernels", "ftq_debug_gemv_plan", "ftq_moe_q4_0_q8_1_noalloc",
)


class FtqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ftq status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libftq.so (built in-tree by quantized_moe_expert_quantize_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FtqError(-1, f"{LIB_PATH} is not built; run `python -m quantized_moe_expert_quantize_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.ftq_quantize_q8_1.argtypes = [P, I64, I64, P, P]
    L.ftq_quantize_q8_1.restype = I32
    L.ftq_quantize_q4_0.argtypes = [P, I64, I64, P, P]
    L.ftq_quantize_q4_0.restype = I32
    L.ftq_moe_select_path.argtypes = [I64, I64, I64, I64, I64]
    L.ftq_moe_select_path.restype = I32
    L.ftq_moe_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I32]
    L.ftq_moe_workspace_bytes.restype = I64
    L.ftq_moe_q4_0_q8_1.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P, SZ, I32, P]
    L.ftq_moe_q4_0_q8_1.restype = I32
    L.ftq_moe_route.argtypes = [P, I64, I64, I64, P, SZ, I32, P]
    L.ftq_moe_route.restype = I32
    L.ftq_moe_q4_0_q8_1_routed.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P, SZ, I32, P]
    L.ftq_moe_q4_0_q8_1_routed.restype = I32
    L.ftq_moe_q4_0_q8_1_partials.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P, SZ, I32, P]
    L.ftq_moe_pairs_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I32]
    L.ftq_moe_pairs_workspace_bytes.restype = I64
    for name in ("ftq_moe_q4_0_q8_1_pairs", "ftq_moe_q4_0_q8_1_pairs_routed", "ftq_moe_q4_0_q8_1_pairs_partials"):
        getattr(L, name).argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P, SZ, I32, P]
        getattr(L, name).restype = I32
    L.ftq_moe_combine_topk.argtypes = [P, P, P, I64, I64, I64, P]
    L.ftq_moe_combine_topk.restype = I32
    for name in ("ftq_moe_q4_0_q8_1_act", "ftq_moe_q4_0_q8_1_act_routed"):
        f = getattr(L, name)
        f.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I32, P, ctypes.c_size_t, I32, P]
        f.restype = I32
    L.ftq_moe_q4_0_q8_1_partials.restype = I32
    for name in ("ftq_moe_gguf_q8_1", "ftq_moe_gguf_q8_1_partials"):
        f = getattr(L, name)
        f.argtypes = [P, I32, P, P, P, I64, I64, I64, I64, I64, I32, P, SZ, I32, P]
        f.restype = I32
    L.ftq_last_error.restype = ctypes.c_char_p
    L.ftq_version.restype = ctypes.c_char_p
    L.ftq_debug_force_block_threads.argtypes = [I32]
    L.ftq_debug_force_block_threads.restype = None
    L.ftq_debug_grouped_kernel.argtypes = [I32]
    L.ftq_debug_grouped_kernel.restype = I32
    L.ftq_debug_route_kernels.argtypes = [I32]
    L.ftq_debug_route_kernels.restype = None
    L.ftq_debug_gemv_plan.argtypes = [I64, I64, I64, I64, I64, I32, I32, P, P, P]
    L.ftq_debug_gemv_plan.restype = I32
    L.ftq_moe_q4_0_q8_1_noalloc.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I32, P]
    L.ftq_moe_q4_0_q8_1_noalloc.restype = I32
    _lib = L
    return L


def last_error() -> str:
    return lib().ftq_last_error().decode()


def version() -> str:
    return lib().ftq_version().decode()


def _check(status: int):
    if status != OK:
        raise FtqError(status, last_error())


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _out(out: torch.Tensor, numel: int, name: str, dtype):
    """A caller's output buffer must hold exactly the elements the call writes."""
    if out.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {out.numel()}")
    return _dev(out, name, dtype)


def quantize_q8_1(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp32 [T, K] -> uint8 [T, K/32*36] Q8_1 blocks."""
    T, K = x.shape
    if out is None:
        out = torch.empty((T, K // QK * Q8_1_BYTES), dtype=torch.uint8, device=x.device)
    _check(lib().ftq_quantize_q8_1(_dev(x, "x", torch.float32), T, K, _out(out, T * (K // QK) * Q8_1_BYTES, "out", torch.uint8),
                                   _stream(stream)))
    return out


def quantize_q4_0(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp32 [..., K] -> uint8 [..., K/32*18] Q4_0 blocks."""
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if out is None:
        out = torch.empty(tuple(w.shape[:-1]) + (K // QK * Q4_0_BYTES,), dtype=torch.uint8, device=w.device)
    _check(lib().ftq_quantize_q4_0(_dev(w, "w", torch.float32), rows, K, _out(out, rows * (K // QK) * Q4_0_BYTES, "out", torch.uint8),
                                   _stream(stream)))
    return out


def gemv_plan(E: int, N: int, K: int, T: int, top_k: int, wtype: int = 2, act: int = 0) -> dict:
    """The GEMV path's on-chip plan for these sizes (host arithmetic): K blocks
    per segment, activation rows per pass, workgroups per CU."""
    seg, pc, per_cu = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ftq_debug_gemv_plan(E, N, K, T, top_k, wtype, act, ctypes.addressof(seg), ctypes.addressof(pc),
                                     ctypes.addressof(per_cu)))
    return {"seg": seg.value, "pairs_per_pass": pc.value, "wg_per_cu": per_cu.value}


def grouped_kernel(variant: int):
    """Select the grouped path's kernel for later calls on this thread
    (GROUPED_I8, GROUPED_F16 or GROUPED_F16_WS)."""
    _check(lib().ftq_debug_grouped_kernel(variant))


def route_kernels(split: bool):
    """Bucketing in three kernels at any size (True) or, for small batches, in
    one workgroup (False, the default) for later calls on this thread."""
    lib().ftq_debug_route_kernels(1 if split else 0)


def select_path(E: int, N: int, K: int, T: int, top_k: int) -> int:
    r = lib().ftq_moe_select_path(E, N, K, T, top_k)
    if r < 0:
        raise FtqError(-r, last_error())
    return r


def workspace_bytes(E: int, N: int, K: int, T: int, top_k: int, path: int = PATH_AUTO) -> int:
    r = lib().ftq_moe_workspace_bytes(E, N, K, T, top_k, path)
    if r < 0:
        raise FtqError(ERR_INVALID_ARG, last_error())
    return r


def _moe_args(w, a, topk_ids, E, N, K, per_pair=False):
    T, top_k = topk_ids.shape
    nb = K // QK
    if w.numel() != E * N * nb * Q4_0_BYTES:
        raise ValueError("w must hold E*N*(K/32) Q4_0 blocks")
    rows = T * top_k if per_pair else T
    if a.numel() != rows * nb * Q8_1_BYTES:
        raise ValueError(f"a must hold {'T*top_k' if per_pair else 'T'}*(K/32) Q8_1 blocks")
    return T, top_k


def _workspace(ws, need, device):
    if need == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if ws.numel() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return ws, ws.numel()


def moe(w: torch.Tensor, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
        path: int = PATH_AUTO, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
        stream=None) -> torch.Tensor:
    """MoE expert matmul: fp32 out [T*top_k, N]."""
    T, top_k = _moe_args(w, a, topk_ids, E, N, K)
    if out is None:
        out = torch.empty((T * top_k, N), dtype=torch.float32, device=a.device)
    need = workspace_bytes(E, N, K, T, top_k, path)
    ws, ws_n = _workspace(workspace, need, a.device)
    _check(lib().ftq_moe_q4_0_q8_1(
        _dev(w, "w", torch.uint8), _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * N, "out", torch.float32), E, N, K, T, top_k,
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


def moe_noalloc(w: torch.Tensor, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
                out: torch.Tensor, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """moe() through ftq_moe_q4_0_q8_1_noalloc: no workspace, the library's
    fixed per-device scratch instead.  `out` is the caller's (nothing here
    allocates device memory)."""
    T, top_k = _moe_args(w, a, topk_ids, E, N, K)
    _check(lib().ftq_moe_q4_0_q8_1_noalloc(
        _dev(w, "w", torch.uint8), _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * N, "out", torch.float32), E, N, K, T, top_k, path, _stream(stream)))
    return out


def moe_route(topk_ids: torch.Tensor, E: int, workspace: torch.Tensor | None, path: int = PATH_AUTO,
              stream=None) -> None:
    """Group the pairs by expert into `workspace` (see ftq_moe_route)."""
    T, top_k = topk_ids.shape
    ws_n = workspace.numel() if workspace is not None else 0
    _check(lib().ftq_moe_route(_dev(topk_ids, "topk_ids", torch.int32), E, T, top_k,
                               workspace.data_ptr() if workspace is not None else None, ws_n, path,
                               _stream(stream)))


def moe_routed(w: torch.Tensor, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
               out: torch.Tensor, workspace: torch.Tensor | None, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """The matmul on pairs already routed into `workspace` by moe_route."""
    T, top_k = _moe_args(w, a, topk_ids, E, N, K)
    ws_n = workspace.numel() if workspace is not None else 0
    _check(lib().ftq_moe_q4_0_q8_1_routed(
        _dev(w, "w", torch.uint8), _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * N, "out", torch.float32), E, N, K, T, top_k,
        workspace.data_ptr() if workspace is not None else None, ws_n, path, _stream(stream)))
    return out


def moe_partials(w: torch.Tensor, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
                 path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """Exact integer block partials int32 [T*top_k, N, K/32]."""
    T, top_k = _moe_args(w, a, topk_ids, E, N, K)
    out = torch.empty((T * top_k, N, K // QK), dtype=torch.int32, device=a.device)
    need = workspace_bytes(E, N, K, T, top_k, path)
    ws, ws_n = _workspace(None, need, a.device)
    _check(lib().ftq_moe_q4_0_q8_1_partials(
        _dev(w, "w", torch.uint8), _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(out, "partials", torch.int32), E, N, K, T, top_k,
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


# ---- per-pair activations (down projection) and the top-k combine -----------

def pairs_workspace_bytes(E: int, N: int, K: int, T: int, top_k: int, path: int = PATH_AUTO) -> int:
    r = lib().ftq_moe_pairs_workspace_bytes(E, N, K, T, top_k, path)
    if r < 0:
        raise FtqError(ERR_INVALID_ARG, last_error())
    return r


def moe_pairs(w: torch.Tensor, a_pairs: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
              path: int = PATH_AUTO, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """MoE expert matmul on per-pair activations a_pairs [T*top_k, K/32 Q8_1 blocks]:
    fp32 out [T*top_k, N]."""
    T, top_k = _moe_args(w, a_pairs, topk_ids, E, N, K, per_pair=True)
    if out is None:
        out = torch.empty((T * top_k, N), dtype=torch.float32, device=a_pairs.device)
    need = pairs_workspace_bytes(E, N, K, T, top_k, path)
    ws, ws_n = _workspace(workspace, need, a_pairs.device)
    _check(lib().ftq_moe_q4_0_q8_1_pairs(
        _dev(w, "w", torch.uint8), _dev(a_pairs, "a_pairs", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * N, "out", torch.float32), E, N, K, T, top_k,
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


def moe_pairs_routed(w: torch.Tensor, a_pairs: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
                     out: torch.Tensor, workspace: torch.Tensor | None, path: int = PATH_AUTO,
                     stream=None) -> torch.Tensor:
    """moe_pairs on pairs already routed into `workspace` (sized by pairs_workspace_bytes) by moe_route."""
    T, top_k = _moe_args(w, a_pairs, topk_ids, E, N, K, per_pair=True)
    ws_n = workspace.numel() if workspace is not None else 0
    _check(lib().ftq_moe_q4_0_q8_1_pairs_routed(
        _dev(w, "w", torch.uint8), _dev(a_pairs, "a_pairs", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * N, "out", torch.float32), E, N, K, T, top_k,
        workspace.data_ptr() if workspace is not None else None, ws_n, path, _stream(stream)))
    return out


def moe_pairs_partials(w: torch.Tensor, a_pairs: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
                       path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """Exact integer block partials int32 [T*top_k, N, K/32] on per-pair activations."""
    T, top_k = _moe_args(w, a_pairs, topk_ids, E, N, K, per_pair=True)
    out = torch.empty((T * top_k, N, K // QK), dtype=torch.int32, device=a_pairs.device)
    need = pairs_workspace_bytes(E, N, K, T, top_k, path)
    ws, ws_n = _workspace(None, need, a_pairs.device)
    _check(lib().ftq_moe_q4_0_q8_1_pairs_partials(
        _dev(w, "w", torch.uint8), _dev(a_pairs, "a_pairs", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(out, "partials", torch.int32), E, N, K, T, top_k,
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


# ---- first layer with the gated activation fused (gate rows, then up rows) ----

def moe_act(w: torch.Tensor, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int, act: int,
            path: int = PATH_AUTO, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """act(gate) * up: fp32 out [T*top_k, N/2] from N = 2*(N/2) weight rows per expert."""
    T, top_k = _moe_args(w, a, topk_ids, E, N, K)
    if out is None:
        out = torch.empty((T * top_k, N // 2), dtype=torch.float32, device=a.device)
    need = workspace_bytes(E, N, K, T, top_k, path)
    ws, ws_n = _workspace(workspace, need, a.device)
    _check(lib().ftq_moe_q4_0_q8_1_act(
        _dev(w, "w", torch.uint8), _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * (N // 2), "out", torch.float32), E, N, K, T, top_k, act,
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


def moe_act_routed(w: torch.Tensor, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int, act: int,
                   out: torch.Tensor, workspace: torch.Tensor | None, path: int = PATH_AUTO,
                   stream=None) -> torch.Tensor:
    """moe_act on pairs already routed into `workspace` by moe_route."""
    T, top_k = _moe_args(w, a, topk_ids, E, N, K)
    ws_n = workspace.numel() if workspace is not None else 0
    _check(lib().ftq_moe_q4_0_q8_1_act_routed(
        _dev(w, "w", torch.uint8), _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * (N // 2), "out", torch.float32), E, N, K, T, top_k, act,
        workspace.data_ptr() if workspace is not None else None, ws_n, path, _stream(stream)))
    return out


# ---- the other GGUF weight block types (GEMV path) ---------------------------

def _gguf_args(w, wtype, a, topk_ids, E, N, K, per_pair):
    T, top_k = topk_ids.shape
    nb = K // QK
    if wtype not in W_BLOCK_BYTES:
        raise ValueError(f"unknown weight type {wtype}")
    if w.numel() != E * N * nb * W_BLOCK_BYTES[wtype]:
        raise ValueError("w must hold E*N*(K/32) blocks of the weight type")
    rows = T * top_k if per_pair else T
    if a.numel() != rows * nb * Q8_1_BYTES:
        raise ValueError(f"a must hold {'T*top_k' if per_pair else 'T'}*(K/32) Q8_1 blocks")
    return T, top_k


def moe_gguf(w: torch.Tensor, wtype: int, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
             per_pair: bool = False, path: int = PATH_AUTO, out: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Matmul with weights of GGUF type `wtype` (W_*): fp32 out [T*top_k, N]."""
    T, top_k = _gguf_args(w, wtype, a, topk_ids, E, N, K, per_pair)
    if out is None:
        out = torch.empty((T * top_k, N), dtype=torch.float32, device=a.device)
    need = workspace_bytes(E, N, K, T, top_k, PATH_GEMV if wtype in GEMV_ONLY else path)
    ws, ws_n = _workspace(workspace, need, a.device)
    _check(lib().ftq_moe_gguf_q8_1(
        _dev(w, "w", torch.uint8), wtype, _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _out(out, T * top_k * N, "out", torch.float32), E, N, K, T, top_k, int(per_pair),
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


def moe_gguf_partials(w: torch.Tensor, wtype: int, a: torch.Tensor, topk_ids: torch.Tensor, E: int, N: int, K: int,
                      per_pair: bool = False, path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """Integer parts sum((q - z) * q8), int32 [T*top_k, N, K/32]."""
    T, top_k = _gguf_args(w, wtype, a, topk_ids, E, N, K, per_pair)
    out = torch.empty((T * top_k, N, K // QK), dtype=torch.int32, device=a.device)
    need = workspace_bytes(E, N, K, T, top_k, PATH_GEMV if wtype in GEMV_ONLY else path)
    ws, ws_n = _workspace(None, need, a.device)
    _check(lib().ftq_moe_gguf_q8_1_partials(
        _dev(w, "w", torch.uint8), wtype, _dev(a, "a", torch.uint8), _dev(topk_ids, "topk_ids", torch.int32),
        _dev(out, "partials", torch.int32), E, N, K, T, top_k, int(per_pair),
        ws.data_ptr() if ws is not None else None, ws_n, path, _stream(stream)))
    return out


def combine_topk(y: torch.Tensor, gates: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[t, n] = sum_j gates[t, j] * y[t*top_k + j, n] (fp32, j ascending)."""
    T, top_k = gates.shape
    if y.dim() != 2 or y.shape[0] != T * top_k:
        raise ValueError("y must be [T*top_k, N]")
    N = y.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=y.device)
    _check(lib().ftq_moe_combine_topk(_dev(y, "y", torch.float32), _dev(gates, "gates", torch.float32),
                                      _out(out, T * N, "out", torch.float32), T, top_k, N, _stream(stream)))
    return out
