"""Python binding of libmsa (ctypes). Argument marshalling only.

Every computation runs in the HIP kernels of libmsa.so; this module checks
tensor shapes, allocates outputs and workspace with torch on the tensors'
device, and passes raw device pointers and torch's current HIP stream across
the C ABI declared in include/msa.h. If libmsa.so is missing or cannot be
loaded, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK = 0
MSA_CAUSAL = 1
MSA_POOLED_VISIBLE_ONLY = 2
(OP_INDEX_SCORES, OP_BLOCK_TOPK, OP_SPARSE_ATTN_FWD, OP_FWD, OP_SPARSE_ATTN_BWD, OP_INDEX_TOPK, OP_DECODE,
 OP_INDEX_BWD) = range(8)

BLOCK_SIZE = 128
HEAD_DIM = 128


class MsaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32),
        ("h_idx", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class MsaError(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func} failed: {message} (status {status})")
        self.status = status


_P = ctypes.c_void_p
_S = ctypes.POINTER(MsaShape)
_SIGNATURES = {
    "msa_workspace_size": [_S, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)],
    "msa_index_scores": [_S, _P, _P, _P, _P],
    "msa_block_topk": [_S, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_sparse_attn_fwd": [_S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_sparse_attn_plan": [_S, _P, _P, ctypes.c_size_t, _P],
    "msa_sparse_attn_partial": [_S, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_sparse_attn_combine": [_S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_fwd": [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_sparse_attn_bwd": [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_index_topk": [_S, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_decode_index_scores": [_S, _P, _P, _P, _P, _P],
    "msa_decode_topk": [_S, _P, _P, _P, _P],
    "msa_decode_attn": [_S, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_decode": [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "msa_decode_noalloc": [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "msa_index_bwd": [_S, _P, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P],
}

_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libmsa.so once. torch is imported first so the library binds to torch's HIP runtime."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_sparse_attention_head_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, args in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.argtypes = args
                    fn.restype = ctypes.c_int
                handle.msa_status_string.argtypes = [ctypes.c_int]
                handle.msa_status_string.restype = ctypes.c_char_p
                _lib = handle
    return _lib


def _check(name: str, status: int) -> None:
    if status != MSA_OK:
        msg = lib().msa_status_string(status).decode()
        raise MsaError(name, status, msg)


def make_shape(batch: int, seqlen: int, h_q: int, h_kv: int, top_k: int, softmax_scale: float,
               h_idx: Optional[int] = None, flags: int = MSA_CAUSAL) -> MsaShape:
    return MsaShape(batch, seqlen, h_q, h_kv, h_kv if h_idx is None else h_idx, HEAD_DIM, HEAD_DIM, BLOCK_SIZE,
                    top_k, float(softmax_scale), flags)


def workspace_size(shape: MsaShape, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("msa_workspace_size", lib().msa_workspace_size(ctypes.byref(shape), op, ctypes.byref(n)))
    return int(n.value)


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def alloc_workspace(shape: MsaShape, op: int, device: torch.device) -> torch.Tensor:
    return torch.empty(max(workspace_size(shape, op), 1), dtype=torch.uint8, device=device)


def _ws(workspace: Optional[torch.Tensor], shape: MsaShape, op: int, device) -> torch.Tensor:
    if workspace is None:
        return alloc_workspace(shape, op, device)
    if workspace.device != torch.device(device) or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    return workspace


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def index_scores(q_idx: torch.Tensor, k_idx: torch.Tensor, pooled: Optional[torch.Tensor] = None,
                 visible_only: bool = False) -> torch.Tensor:
    """Pooled index scores fp32 [B, H_idx, N, N/128] (see msa_index_scores)."""
    B, N, H, D = q_idx.shape
    _need(q_idx, "q_idx", torch.bfloat16, (B, N, H, D))
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, D))
    nblk = -(-N // BLOCK_SIZE)
    if pooled is None:
        pooled = torch.empty((B, H, N, nblk), dtype=torch.float32, device=q_idx.device)
    _need(pooled, "pooled", torch.float32, (B, H, N, nblk))
    flags = MSA_CAUSAL | (MSA_POOLED_VISIBLE_ONLY if visible_only else 0)
    shape = make_shape(B, N, H, H, 1, 1.0, flags=flags)
    _check("msa_index_scores", lib().msa_index_scores(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(pooled),
                                                      _stream(q_idx.device)))
    return pooled


def block_topk(pooled: torch.Tensor, top_k: int, block_idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Selected blocks int32 [B, H_idx, N, top_k] from pooled scores (see msa_block_topk)."""
    B, H, N, nblk = pooled.shape
    _need(pooled, "pooled", torch.float32, (B, H, N, nblk))
    if block_idx is None:
        block_idx = torch.empty((B, H, N, top_k), dtype=torch.int32, device=pooled.device)
    _need(block_idx, "block_idx", torch.int32, (B, H, N, top_k))
    shape = make_shape(B, N, H, H, top_k, 1.0)
    _check("msa_block_topk", lib().msa_block_topk(ctypes.byref(shape), _ptr(pooled), _ptr(block_idx), _P(0), 0,
                                                  _stream(pooled.device)))
    return block_idx


def index_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, top_k: int, block_idx: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """block_idx int32 [B, H_idx, N, top_k]: index scores and selection in one step (see msa_index_topk)."""
    B, N, H, D = q_idx.shape
    _need(q_idx, "q_idx", torch.bfloat16, (B, N, H, D))
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, D))
    if block_idx is None:
        block_idx = torch.empty((B, H, N, top_k), dtype=torch.int32, device=q_idx.device)
    _need(block_idx, "block_idx", torch.int32, (B, H, N, top_k))
    shape = make_shape(B, N, H, H, top_k, 1.0)
    ws = _ws(workspace, shape, OP_INDEX_TOPK, q_idx.device)
    _check("msa_index_topk", lib().msa_index_topk(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                                                  _ptr(ws), ws.numel(), _stream(q_idx.device)))
    return block_idx


def _attn_shape(q, k, v, block_idx, softmax_scale) -> MsaShape:
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    top_k = block_idx.shape[-1]
    _need(q, "q", torch.bfloat16, (B, N, Hq, D))
    _need(k, "k", torch.bfloat16, (B, N, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, N, Hkv, D))
    _need(block_idx, "block_idx", torch.int32, (B, Hkv, N, top_k))
    return make_shape(B, N, Hq, Hkv, top_k, softmax_scale)


def sparse_attn_fwd(q, k, v, block_idx, softmax_scale: float, o=None, lse=None, workspace=None):
    """(O bf16 [B,N,H_q,128], LSE fp32 [B,H_q,N]) over the selected blocks (see msa_sparse_attn_fwd)."""
    shape = _attn_shape(q, k, v, block_idx, softmax_scale)
    B, N, Hq, D = q.shape
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "o", torch.bfloat16, (B, N, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq, N))
    ws = _ws(workspace, shape, OP_SPARSE_ATTN_FWD, q.device)
    _check("msa_sparse_attn_fwd",
           lib().msa_sparse_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(o),
                                     _ptr(lse), _ptr(ws), ws.numel(), _stream(q.device)))
    return o, lse


def sparse_attn_bwd(q, k, v, o, lse, d_o, block_idx, softmax_scale: float, dq=None, dk=None, dv=None,
                    workspace=None):
    """(dQ, dK, dV) in bf16 over the cached selection (see msa_sparse_attn_bwd)."""
    shape = _attn_shape(q, k, v, block_idx, softmax_scale)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    _need(o, "o", torch.bfloat16, (B, N, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq, N))
    _need(d_o, "d_o", torch.bfloat16, (B, N, Hq, D))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, (B, N, Hq, D))
    _need(dk, "dk", torch.bfloat16, (B, N, Hkv, D))
    _need(dv, "dv", torch.bfloat16, (B, N, Hkv, D))
    ws = _ws(workspace, shape, OP_SPARSE_ATTN_BWD, q.device)
    _check("msa_sparse_attn_bwd",
           lib().msa_sparse_attn_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o),
                                     _ptr(block_idx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                                     _stream(q.device)))
    return dq, dk, dv


def index_bwd(q_idx, k_idx, q, k, lse, block_idx, softmax_scale: float, index_scale: Optional[float] = None,
              kl_weight: float = 1.0, dq_idx=None, dk_idx=None, workspace=None):
    """(dq_idx bf16 [B,N,H_idx,128], dk_idx bf16 [B,N,128]): the index branch's KL gradient (see msa_index_bwd)."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    shape = _attn_shape(q, k, k, block_idx, softmax_scale)
    _need(q_idx, "q_idx", torch.bfloat16, (B, N, Hkv, D))
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, D))
    _need(lse, "lse", torch.float32, (B, Hq, N))
    dq_idx = torch.empty_like(q_idx) if dq_idx is None else dq_idx
    dk_idx = torch.empty_like(k_idx) if dk_idx is None else dk_idx
    _need(dq_idx, "dq_idx", torch.bfloat16, (B, N, Hkv, D))
    _need(dk_idx, "dk_idx", torch.bfloat16, (B, N, D))
    ws = _ws(workspace, shape, OP_INDEX_BWD, q.device)
    s_idx = softmax_scale if index_scale is None else index_scale
    _check("msa_index_bwd", lib().msa_index_bwd(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k),
                                                _ptr(lse), _ptr(block_idx), float(s_idx), float(kl_weight),
                                                _ptr(dq_idx), _ptr(dk_idx), _ptr(ws), ws.numel(), _stream(q.device)))
    return dq_idx, dk_idx


def sparse_attn_plan(shape: MsaShape, block_idx: torch.Tensor, workspace: torch.Tensor) -> None:
    _check("msa_sparse_attn_plan", lib().msa_sparse_attn_plan(ctypes.byref(shape), _ptr(block_idx), _ptr(workspace),
                                                              workspace.numel(), _stream(block_idx.device)))


def sparse_attn_partial(shape: MsaShape, q, k, v, workspace: torch.Tensor) -> None:
    _check("msa_sparse_attn_partial",
           lib().msa_sparse_attn_partial(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(workspace),
                                         workspace.numel(), _stream(q.device)))


def sparse_attn_combine(shape: MsaShape, q, k, v, block_idx, o, lse, workspace: torch.Tensor) -> None:
    """Merge of the slot partials into o and lse; q, k, v are read for the queries' own blocks."""
    _check("msa_sparse_attn_combine",
           lib().msa_sparse_attn_combine(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(o),
                                         _ptr(lse), _ptr(workspace), workspace.numel(), _stream(o.device)))


def msa_fwd(q_idx, k_idx, q, k, v, top_k: int, softmax_scale: float, block_idx=None, o=None, lse=None,
            workspace=None):
    """The whole forward; returns (block_idx int32 [B,H_kv,N,top_k], O, LSE) (see msa_fwd)."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    _need(q_idx, "q_idx", torch.bfloat16, (B, N, Hkv, D))
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, D))
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, N, top_k), dtype=torch.int32, device=q.device)
    shape = _attn_shape(q, k, v, block_idx, softmax_scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "o", torch.bfloat16, (B, N, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq, N))
    ws = _ws(workspace, shape, OP_FWD, q.device)
    _check("msa_fwd", lib().msa_fwd(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q.device)))
    return block_idx, o, lse


# ---------------------------------------------------------------------------
# Decode: one new query per sequence against its caches (see the decode calls in msa.h)
# ---------------------------------------------------------------------------
def _decode_shape(q_idx, k_idx, q, k, v, seqlens, top_k: int, softmax_scale: float) -> MsaShape:
    B, H, D = q_idx.shape
    C = k_idx.shape[1]
    Hq = q.shape[1]
    Hkv = k.shape[2]
    _need(q_idx, "q_idx", torch.bfloat16, (B, H, D))
    _need(k_idx, "k_idx", torch.bfloat16, (B, C, D))
    _need(q, "q", torch.bfloat16, (B, Hq, D))
    _need(k, "k", torch.bfloat16, (B, C, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, C, Hkv, D))
    _need(seqlens, "seqlens", torch.int32, (B,))
    if H != Hkv:
        raise ValueError("one index head per KV head")
    return make_shape(B, C, Hq, Hkv, top_k, softmax_scale)


def decode_index_scores(q_idx, k_idx, seqlens, pooled=None) -> torch.Tensor:
    """pooled fp32 [B, H_idx, C/128] of the new token (see msa_decode_index_scores)."""
    B, H, D = q_idx.shape
    C = k_idx.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16, (B, H, D))
    _need(k_idx, "k_idx", torch.bfloat16, (B, C, D))
    _need(seqlens, "seqlens", torch.int32, (B,))
    nb = C // 128
    pooled = torch.empty((B, H, nb), dtype=torch.float32, device=q_idx.device) if pooled is None else pooled
    _need(pooled, "pooled", torch.float32, (B, H, nb))
    shape = make_shape(B, C, H, H, 1, 1.0)
    _check("msa_decode_index_scores", lib().msa_decode_index_scores(
        ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(seqlens), _ptr(pooled), _stream(q_idx.device)))
    return pooled


def decode_topk(pooled, seqlens, top_k: int, capacity: int, block_idx=None) -> torch.Tensor:
    """block_idx int32 [B, H_idx, top_k] (see msa_decode_topk)."""
    B, H, nb = pooled.shape
    _need(pooled, "pooled", torch.float32, (B, H, capacity // 128))
    _need(seqlens, "seqlens", torch.int32, (B,))
    block_idx = torch.empty((B, H, top_k), dtype=torch.int32, device=pooled.device) if block_idx is None \
        else block_idx
    _need(block_idx, "block_idx", torch.int32, (B, H, top_k))
    shape = make_shape(B, capacity, H, H, top_k, 1.0)
    _check("msa_decode_topk", lib().msa_decode_topk(ctypes.byref(shape), _ptr(pooled), _ptr(seqlens),
                                                    _ptr(block_idx), _stream(pooled.device)))
    return block_idx


def decode_attn(q, k, v, seqlens, block_idx, softmax_scale: float, o=None, lse=None, workspace=None):
    """(O bf16 [B, H_q, 128], LSE fp32 [B, H_q]) over the selected blocks (see msa_decode_attn).
    With a workspace (uint8, msa_workspace_size(MSA_OP_DECODE) bytes) a step with few sequences
    spreads each group's blocks over several workgroups, as msa_decode does."""
    B, Hq, D = q.shape
    C, Hkv = k.shape[1], k.shape[2]
    top_k = block_idx.shape[-1]
    _need(q, "q", torch.bfloat16, (B, Hq, D))
    _need(k, "k", torch.bfloat16, (B, C, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, C, Hkv, D))
    _need(seqlens, "seqlens", torch.int32, (B,))
    _need(block_idx, "block_idx", torch.int32, (B, Hkv, top_k))
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "o", torch.bfloat16, (B, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq))
    shape = make_shape(B, C, Hq, Hkv, top_k, softmax_scale)
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()
                                  or workspace.device != q.device):
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    _check("msa_decode_attn", lib().msa_decode_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens), _ptr(block_idx), _ptr(o), _ptr(lse),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q.device)))
    return o, lse


def decode(q_idx, k_idx, q, k, v, seqlens, top_k: int, softmax_scale: float, block_idx=None, o=None, lse=None,
           workspace=None):
    """(block_idx [B, H_idx, top_k], O [B, H_q, 128], LSE [B, H_q]) of one decode step (see msa_decode)."""
    shape = _decode_shape(q_idx, k_idx, q, k, v, seqlens, top_k, softmax_scale)
    B, H, _ = q_idx.shape
    Hq = q.shape[1]
    block_idx = torch.empty((B, H, top_k), dtype=torch.int32, device=q.device) if block_idx is None else block_idx
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(block_idx, "block_idx", torch.int32, (B, H, top_k))
    _need(o, "o", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq))
    ws = _ws(workspace, shape, OP_DECODE, q.device)
    _check("msa_decode", lib().msa_decode(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(seqlens), _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                          _stream(q.device)))
    return block_idx, o, lse


def decode_noalloc(q_idx, k_idx, q, k, v, seqlens, top_k: int, softmax_scale: float, block_idx=None, o=None,
                   lse=None):
    """msa_decode_noalloc: the decode step with the library's static scratch (no workspace).
    Outputs are allocated here only when not given; pass them to keep the call allocation-free."""
    shape = _decode_shape(q_idx, k_idx, q, k, v, seqlens, top_k, softmax_scale)
    B, H, _ = q_idx.shape
    Hq = q.shape[1]
    block_idx = torch.empty((B, H, top_k), dtype=torch.int32, device=q.device) if block_idx is None else block_idx
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(block_idx, "block_idx", torch.int32, (B, H, top_k))
    _need(o, "o", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq))
    _check("msa_decode_noalloc", lib().msa_decode_noalloc(
        ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens), _ptr(block_idx),
        _ptr(o), _ptr(lse), _stream(q.device)))
    return block_idx, o, lse
