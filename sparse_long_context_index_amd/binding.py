"""ctypes binding of libdsa.so (argument marshalling only).

Every function here forwards device pointers, sizes and the current torch
stream to the C ABI declared in include/dsa.h; all arithmetic runs in the HIP
kernels.  There is no fallback: if the library is missing, or a tensor is not
on a GPU, the call raises.

Functions carry the C names: dsa_index_scores, dsa_topk, sparse_gqa_attn,
swa_attn, dsa_decode_step, dsa_cache_append, plus the workspace helpers.  Tensors are torch
tensors on the GPU with the layouts of dsa.h (uint8 for fp8 bytes, bfloat16
or int16/uint16 for bf16, float32, int32, int64).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK = 0
STATUS = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_UNSUPPORTED",
          4: "DSA_ERR_ALIGN", 5: "DSA_ERR_WORKSPACE", 6: "DSA_ERR_HIP", 7: "DSA_ERR_SCRATCH"}
STATIC_SCRATCH_BYTES = 64 << 20      # DSA_STATIC_SCRATCH_BYTES
OP_INDEX_SCORES, OP_TOPK, OP_SPARSE_ATTN, OP_SWA_ATTN, OP_DECODE_STEP, OP_PREFILL_TOPK, OP_DECODE_BATCH, \
    OP_INDEX_RECALL = range(8)

IDX_HEADS, IDX_DIM, Q_HEADS, QK_DIM, V_DIM = 16, 128, 64, 192, 128
KV_HEADS, SWA_KV_HEADS = 4, 8
ROPE_BASE = 1.0e7          # DSA_ROPE_BASE
ROT_IDX, ROT_MAIN = 42, 64  # a third of the 128- and 192-dim heads
DSA_KV_HEADS, SWA_KV_HEADS, TOPK_MAX, DECODE_T_MAX = 4, 8, 2048, 8

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "dsa_index_scores": ([_P, _P, _P, _I64, _I32, _P, _I64, _P], _I32),
    "dsa_topk": ([_P, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P], _I32),
    "sparse_gqa_attn": ([_P, _P, _P, _I64, _P, _I32, _I32, _P, _F, _P, _P, _P, _SZ, _P], _I32),
    "swa_attn": ([_P, _P, _P, _I64, _P, _P, _I32, _I32, _P, _F, _P, _P, _P, _SZ, _P], _I32),
    "dsa_decode_step": ([_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _P, _F, _P, _P, _P, _P, _I64,
                         _P, _SZ, _P], _I32),
    "dsa_decode_step_noalloc": ([_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _P, _F, _P, _P, _P, _P, _I64, _P],
                                _I32),
    "dsa_cache_append": ([_P, _P, _P, _P, _F, _P, _P, _P, _I64, _I32, _I32, _I32, ctypes.c_double,
                          _P, _P, _P, _P, _P, _P], _I32),
    "dsa_prefill_topk": ([_P, _P, _P, _I64, _I32, _I32, _P, _P, _SZ, _P], _I32),
    "dsa_decode_batch": ([_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I64, _I32, _P, _F, _P, _P, _P,
                          _P, _SZ, _P], _I32),
    "dsa_index_recall": ([_P, _P, _P, _I64, _P, _I32, _I32, _F, _P, _P, _P, _SZ, _P], _I32),
    "dsa_workspace_bytes": ([_I32, _I64, _I32, _I32, _I32], _SZ),
    "dsa_workspace_init": ([_P, _SZ, _P], _I32),
    "dsa_status_string": ([_I32], ctypes.c_char_p),
    "dsa_version": ([], ctypes.c_char_p),
}

_lib = None


class DsaError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load libdsa.so (built by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise DsaError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != DSA_OK:
        msg = load().dsa_status_string(status).decode()
        raise DsaError(f"{what}: {msg}")


def _dev(t: Optional[torch.Tensor], name: str, need: int = 0):
    """Device pointer of t; need: the bytes the call reads or writes there
    (the C interface takes no buffer sizes, so a short buffer is refused here)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise DsaError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise DsaError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < need:
        raise DsaError(f"{name} holds {t.numel() * t.element_size()} bytes, the call needs {need}")
    return ctypes.c_void_p(t.data_ptr())


def _rows(T: int, ld: int, n: int, item: int = 4) -> int:
    """bytes of T rows of n items at stride ld"""
    return ((T - 1) * ld + n) * item if T > 0 and n > 0 else 0


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(op: int, Lk: int = 0, T: int = 0, k: int = 0, B: int = 0) -> int:
    return int(load().dsa_workspace_bytes(op, Lk, T, k, B))


class Workspace:
    """A device workspace prepared with dsa_workspace_init (grows on demand)."""

    def __init__(self, nbytes: int = 0, device=None):
        self.device = device or torch.device("cuda", torch.cuda.current_device())
        self.buf = None
        if nbytes:
            self.ensure(nbytes)

    def ensure(self, nbytes: int):
        """Grow to at least nbytes (a size from workspace_bytes); a new buffer
        is prepared with dsa_workspace_init."""
        if self.buf is not None and self.buf.numel() >= nbytes:
            return self
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        _check(load().dsa_workspace_init(_dev(self.buf, "ws"), nbytes, _stream()), "dsa_workspace_init")
        return self

    @property
    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())

    @property
    def nbytes(self) -> int:
        return self.buf.numel()


def dsa_index_scores(q_idx, w, k_idx, Lk: int, T: int, scores=None, ld: Optional[int] = None):
    if scores is None:
        scores = torch.empty((T, Lk), dtype=torch.float32, device=q_idx.device)
    ld = scores.shape[-1] if ld is None else ld
    _check(load().dsa_index_scores(_dev(q_idx, "q_idx", T * IDX_HEADS * IDX_DIM), _dev(w, "w", T * IDX_HEADS * 4),
                                   _dev(k_idx, "k_idx", Lk * IDX_DIM), Lk, T,
                                   _dev(scores, "scores", _rows(T, ld, Lk)), ld, _stream()), "dsa_index_scores")
    return scores


def dsa_topk(scores, Lk: int, T: int, k: int, idx=None, ws: Optional[Workspace] = None,
             ld: Optional[int] = None):
    ld = scores.shape[-1] if ld is None else ld
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    ws = (ws or Workspace(device=scores.device)).ensure(workspace_bytes(OP_TOPK, Lk, T, k))
    _check(load().dsa_topk(_dev(scores, "scores", _rows(T, ld, Lk)), ld, Lk, T, k, _dev(idx, "idx", T * k * 4),
                           ws.ptr, ws.nbytes, _stream()), "dsa_topk")
    return idx


def dsa_decode_batch(q_idx, w, k_idx, q, k_cache, v_cache, seq_start, seq_len, max_len: int, k: int, sink,
                     sm_scale: float, out=None, lse=None, idx_out=None, ws: Optional[Workspace] = None):
    """Decode step of B ragged sequences sharing one cache; q_idx [B,T,16,128]."""
    B, T = int(q_idx.shape[0]), int(q_idx.shape[1])
    n_rows = int(k_idx.shape[0])
    if out is None:
        out = torch.empty((B, T, Q_HEADS, V_DIM), dtype=torch.bfloat16, device=q.device)
    ws = (ws or Workspace(device=q.device)).ensure(workspace_bytes(OP_DECODE_BATCH, max_len, T, k, B))
    R = B * T
    _check(load().dsa_decode_batch(_dev(q_idx, "q_idx", R * IDX_HEADS * IDX_DIM), _dev(w, "w", R * IDX_HEADS * 4),
                                   _dev(k_idx, "k_idx", n_rows * IDX_DIM), _dev(q, "q", R * Q_HEADS * QK_DIM * 2),
                                   _dev(k_cache, "k_cache", n_rows * KV_HEADS * QK_DIM * 2),
                                   _dev(v_cache, "v_cache", n_rows * KV_HEADS * V_DIM * 2), n_rows,
                                   _dev(seq_start, "seq_start", B * 8), _dev(seq_len, "seq_len", B * 4), B, T,
                                   max_len, k, _dev(sink, "sink", Q_HEADS * 4), float(sm_scale),
                                   _dev(out, "out", R * Q_HEADS * V_DIM * 2), _dev(lse, "lse", R * Q_HEADS * 4),
                                   _dev(idx_out, "idx_out", R * k * 4), ws.ptr, ws.nbytes, _stream()),
           "dsa_decode_batch")
    return out


def dsa_index_recall(q, k_cache, v_cache, Lk: int, idx, sm_scale: float, recall=None, lse_dense=None,
                     ws: Optional[Workspace] = None):
    """Share of each head's dense softmax mass on the keys idx [T,k] selects."""
    T, k = int(idx.shape[0]), int(idx.shape[1])
    if recall is None:
        recall = torch.empty((T, Q_HEADS), dtype=torch.float32, device=q.device)
    ws = (ws or Workspace(device=q.device)).ensure(workspace_bytes(OP_INDEX_RECALL, Lk, T, k))
    _check(load().dsa_index_recall(_dev(q, "q", T * Q_HEADS * QK_DIM * 2),
                                   _dev(k_cache, "k_cache", Lk * KV_HEADS * QK_DIM * 2),
                                   _dev(v_cache, "v_cache", Lk * KV_HEADS * V_DIM * 2), Lk,
                                   _dev(idx, "idx", T * k * 4), T, k, float(sm_scale),
                                   _dev(recall, "recall", T * Q_HEADS * 4), _dev(lse_dense, "lse_dense", T * Q_HEADS * 4),
                                   ws.ptr, ws.nbytes, _stream()), "dsa_index_recall")
    return recall


def dsa_prefill_topk(q_idx, w, k_idx, Lk: int, T: int, k: int, idx=None, ws: Optional[Workspace] = None):
    """Index scores and per-row top-k of T query rows without the score matrix."""
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=q_idx.device)
    ws = (ws or Workspace(device=q_idx.device)).ensure(workspace_bytes(OP_PREFILL_TOPK, Lk, T, k))
    _check(load().dsa_prefill_topk(_dev(q_idx, "q_idx", T * IDX_HEADS * IDX_DIM), _dev(w, "w", T * IDX_HEADS * 4),
                                   _dev(k_idx, "k_idx", Lk * IDX_DIM), Lk, T, k, _dev(idx, "idx", T * k * 4),
                                   ws.ptr, ws.nbytes, _stream()), "dsa_prefill_topk")
    return idx


def sparse_gqa_attn(q, k_cache, v_cache, Lk: int, idx, sink, sm_scale: float, out=None, lse=None,
                    ws: Optional[Workspace] = None):
    T, k = idx.shape
    if out is None:
        out = torch.empty((T, Q_HEADS, V_DIM), dtype=torch.bfloat16, device=q.device)
    ws = (ws or Workspace(device=q.device)).ensure(workspace_bytes(OP_SPARSE_ATTN, Lk, T, k))
    _check(load().sparse_gqa_attn(_dev(q, "q", T * Q_HEADS * QK_DIM * 2),
                                  _dev(k_cache, "k_cache", Lk * KV_HEADS * QK_DIM * 2),
                                  _dev(v_cache, "v_cache", Lk * KV_HEADS * V_DIM * 2), Lk,
                                  _dev(idx, "idx", T * k * 4), T, k, _dev(sink, "sink", Q_HEADS * 4), float(sm_scale),
                                  _dev(out, "out", T * Q_HEADS * V_DIM * 2), _dev(lse, "lse", T * Q_HEADS * 4),
                                  ws.ptr, ws.nbytes, _stream()),
           "sparse_gqa_attn")
    return out


def swa_attn(q, k_cache, v_cache, seq_start, seq_len, window: int, sink, sm_scale: float, out=None,
             lse=None, ws: Optional[Workspace] = None):
    B = seq_len.shape[0]
    if out is None:
        out = torch.empty((B, Q_HEADS, V_DIM), dtype=torch.bfloat16, device=q.device)
    ws = (ws or Workspace(device=q.device)).ensure(workspace_bytes(OP_SWA_ATTN, B=B))
    n_rows = k_cache.shape[0]
    _check(load().swa_attn(_dev(q, "q", B * Q_HEADS * QK_DIM * 2),
                           _dev(k_cache, "k_cache", n_rows * SWA_KV_HEADS * QK_DIM * 2),
                           _dev(v_cache, "v_cache", n_rows * SWA_KV_HEADS * V_DIM * 2), n_rows,
                           _dev(seq_start, "seq_start", B * 8), _dev(seq_len, "seq_len", B * 4), B,
                           window, _dev(sink, "sink", Q_HEADS * 4), float(sm_scale),
                           _dev(out, "out", B * Q_HEADS * V_DIM * 2), _dev(lse, "lse", B * Q_HEADS * 4),
                           ws.ptr, ws.nbytes, _stream()), "swa_attn")
    return out


def dsa_decode_step(q_idx, w, k_idx, q, k_cache, v_cache, Lk: int, T: int, k: int, sink,
                    sm_scale: float, out=None, lse=None, idx_out=None, scores_out=None,
                    ws: Optional[Workspace] = None):
    if out is None:
        out = torch.empty((T, Q_HEADS, V_DIM), dtype=torch.bfloat16, device=q.device)
    ws = (ws or Workspace(device=q.device)).ensure(workspace_bytes(OP_DECODE_STEP, Lk, T, k))
    args = _step_args(q_idx, w, k_idx, q, k_cache, v_cache, Lk, T, k, sink, sm_scale, out, lse, idx_out, scores_out)
    _check(load().dsa_decode_step(*args, ws.ptr, ws.nbytes, _stream()), "dsa_decode_step")
    return out


def _step_args(q_idx, w, k_idx, q, k_cache, v_cache, Lk, T, k, sink, sm_scale, out, lse, idx_out, scores_out):
    ld = scores_out.shape[-1] if scores_out is not None else 0
    return (_dev(q_idx, "q_idx", T * IDX_HEADS * IDX_DIM), _dev(w, "w", T * IDX_HEADS * 4),
            _dev(k_idx, "k_idx", Lk * IDX_DIM), _dev(q, "q", T * Q_HEADS * QK_DIM * 2),
            _dev(k_cache, "k_cache", Lk * KV_HEADS * QK_DIM * 2), _dev(v_cache, "v_cache", Lk * KV_HEADS * V_DIM * 2),
            Lk, T, k, _dev(sink, "sink", Q_HEADS * 4), float(sm_scale), _dev(out, "out", T * Q_HEADS * V_DIM * 2),
            _dev(lse, "lse", T * Q_HEADS * 4), _dev(idx_out, "idx_out", T * k * 4),
            _dev(scores_out, "scores_out", _rows(T, ld, Lk)), ld)


def dsa_decode_step_noalloc(q_idx, w, k_idx, q, k_cache, v_cache, Lk: int, T: int, k: int, sink,
                            sm_scale: float, out, lse=None, idx_out=None, scores_out=None):
    """dsa_decode_step on the library's static per-GPU scratch: no workspace,
    and the C call allocates nothing (the caller passes every output)."""
    args = _step_args(q_idx, w, k_idx, q, k_cache, v_cache, Lk, T, k, sink, sm_scale, out, lse, idx_out, scores_out)
    _check(load().dsa_decode_step_noalloc(*args, _stream()), "dsa_decode_step_noalloc")
    return out


def dsa_cache_append(idx_q, idx_k, q, k, v, Lk: int, T: int, k_idx_cache, k_cache, v_cache,
                     ln_gamma=None, ln_beta=None, ln_eps: float = 1e-6, rot_idx: int = ROT_IDX,
                     rot_main: int = ROT_MAIN, rope_base: float = ROPE_BASE, q_idx_out=None, q_out=None):
    """Append T new tokens (positions Lk-T .. Lk-1) to the index-key and K/V
    caches; returns (q_idx_out [T,16,128] uint8, q_out [T,64,192] bf16)."""
    dev = idx_q.device
    if q_idx_out is None:
        q_idx_out = torch.empty((T, IDX_HEADS, IDX_DIM), dtype=torch.uint8, device=dev)
    if q_out is None:
        q_out = torch.empty((T, Q_HEADS, QK_DIM), dtype=torch.bfloat16, device=dev)
    _check(load().dsa_cache_append(_dev(idx_q, "idx_q", T * IDX_HEADS * IDX_DIM * 2), _dev(idx_k, "idx_k", T * IDX_DIM * 2),
                                   _dev(ln_gamma, "ln_gamma", IDX_DIM * 4), _dev(ln_beta, "ln_beta", IDX_DIM * 4),
                                   ln_eps, _dev(q, "q", T * Q_HEADS * QK_DIM * 2), _dev(k, "k", T * KV_HEADS * QK_DIM * 2),
                                   _dev(v, "v", T * KV_HEADS * V_DIM * 2), Lk, T, rot_idx, rot_main, rope_base,
                                   _dev(q_idx_out, "q_idx_out", T * IDX_HEADS * IDX_DIM),
                                   _dev(k_idx_cache, "k_idx_cache", Lk * IDX_DIM),
                                   _dev(q_out, "q_out", T * Q_HEADS * QK_DIM * 2),
                                   _dev(k_cache, "k_cache", Lk * KV_HEADS * QK_DIM * 2),
                                   _dev(v_cache, "v_cache", Lk * KV_HEADS * V_DIM * 2), _stream()), "dsa_cache_append")
    return q_idx_out, q_out
