"""DeepSeek Sparse Attention (DSA) hot path on AMD MI355X -- Python binding of libdsa.so.

Argument marshalling only: every step of the path runs in the HIP kernels of libdsa.so,
reached through its C ABI (include/dsa.h).  PyTorch supplies device memory and the stream
(``torch.cuda.current_stream()``).  There is no fallback: if the library cannot be loaded,
every call raises.

Tensor conventions (all on the GPU, contiguous):
    q8 [T,H_I,128] uint8 (OCP e4m3fn codes), q_scale/w [T,H_I] float32,
    k8 [L,128] uint8, k_scale [L] float32, q [T,H,576] bfloat16, kv [L,576] bfloat16,
    scores [T,>=L] float32, idx [T,k] int32, out [T,H,512] bfloat16, lse [T,H] float32.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")
_lock = threading.Lock()
_lib = None

DSA_OK, DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED = 0, 1, 2
DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP = 3, 4

EXPORTS = ("dsa_status_string", "dsa_version", "dsa_index_scores", "dsa_topk",
           "dsa_topk_workspace_bytes", "dsa_sparse_mla", "dsa_prefill",
           "dsa_prefill_workspace_bytes", "dsa_prefill_chunk_rows", "dsa_decode",
           "dsa_decode_workspace_bytes", "dsa_quantize_fp8", "dsa_decode_append",
           "dsa_window_indices", "dsa_local_selected_indices", "dsa_prefill_varlen",
           "dsa_prefill_varlen_workspace_bytes", "dsa_attention_lse",
           "dsa_attention_distribution", "dsa_indexer_warmup", "dsa_indexer_warmup_workspace_bytes",
           "dsa_decode_noalloc", "dsa_decode_noalloc_scratch_bytes")


class DSAError(RuntimeError):
    def __init__(self, status: int, name: str, where: str):
        super().__init__("%s: %s (%d)" % (where, name, status))
        self.status = status


def load(path: str = LIB_PATH):
    """Load libdsa.so (built in-tree by ``build.py``); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("libdsa.so not built: run python -m sparse_attention_05_amd.build")
            lib = ctypes.CDLL(path)
            P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_float, ctypes.c_size_t)
            lib.dsa_status_string.restype = ctypes.c_char_p
            lib.dsa_status_string.argtypes = [i32]
            lib.dsa_version.restype = i32
            lib.dsa_index_scores.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f32, P, i64, i32, P]
            lib.dsa_topk.argtypes = [P, i64, i32, i32, i32, i32, P, P, sz, P]
            lib.dsa_topk_workspace_bytes.restype = sz
            lib.dsa_topk_workspace_bytes.argtypes = [i32, i32, i32]
            lib.dsa_sparse_mla.argtypes = [P, P, P, i32, i32, i32, i32, f32, P, P, P]
            lib.dsa_prefill.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32,
                                        f32, P, P, P, P, sz, P]
            lib.dsa_prefill_workspace_bytes.restype = sz
            lib.dsa_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
            lib.dsa_prefill_chunk_rows.restype = i32
            lib.dsa_prefill_chunk_rows.argtypes = [i32, i32]
            lib.dsa_decode.argtypes = [i32, P, i32, i64, P, P, P, P, P, P, P, i32, i32, i32, f32,
                                       f32, P, P, P, P, sz, P]
            lib.dsa_decode_workspace_bytes.restype = sz
            lib.dsa_decode_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
            lib.dsa_decode_noalloc.argtypes = [i32, P, i32, i64, P, P, P, P, P, P, P, i32, i32,
                                               i32, f32, f32, P, P, P, P]
            lib.dsa_decode_noalloc_scratch_bytes.restype = sz
            lib.dsa_decode_noalloc_scratch_bytes.argtypes = []
            lib.dsa_quantize_fp8.argtypes = [P, i32, i64, P, P, P]
            lib.dsa_decode_append.argtypes = [i32, P, P, i32, P, P, P, P, P]
            lib.dsa_window_indices.argtypes = [i32, i32, i32, i32, P, P]
            lib.dsa_local_selected_indices.argtypes = [P, i32, i32, i32, i32, i32, P, P]
            lib.dsa_prefill_varlen.argtypes = [i32, P, P, P, P, P, P, P, P, P, i32, i32, i32,
                                               f32, f32, P, P, P, P, sz, P]
            lib.dsa_prefill_varlen_workspace_bytes.restype = sz
            lib.dsa_prefill_varlen_workspace_bytes.argtypes = [i32, P, P, i32, i32, i32]
            lib.dsa_attention_lse.argtypes = [P, P, i32, i32, i32, i32, f32, P, P]
            lib.dsa_attention_distribution.argtypes = [P, P, P, i32, i32, i32, i32, f32, P, i64, P]
            lib.dsa_indexer_warmup.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, f32,
                                               f32, P, P, P, P, P, P, P, sz, P]
            lib.dsa_indexer_warmup_workspace_bytes.restype = sz
            lib.dsa_indexer_warmup_workspace_bytes.argtypes = [i32, i32, i32, i32]
            # entry points that return a dsa_status_t (the *_workspace_bytes queries return
            # size_t and are set above)
            for fn in ("dsa_index_scores", "dsa_topk", "dsa_sparse_mla", "dsa_prefill",
                       "dsa_decode", "dsa_decode_noalloc", "dsa_quantize_fp8", "dsa_decode_append",
                       "dsa_window_indices", "dsa_local_selected_indices", "dsa_prefill_varlen",
                       "dsa_attention_lse", "dsa_attention_distribution", "dsa_indexer_warmup"):
                getattr(lib, fn).restype = i32
            _lib = lib
    return _lib


def _check(status: int, where: str):
    if status != DSA_OK:
        raise DSAError(status, load().dsa_status_string(status).decode(), where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _req(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _rows(t, T, L, name):
    """A float32 CUDA matrix of T rows of at least L entries, unit column stride (scores, P)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] != T or t.shape[1] < L \
            or t.stride(1) != 1 or (T > 1 and t.stride(0) < t.shape[1]):
        raise ValueError("%s must be float32 [T, >=L] with unit column stride" % name)
    return t


def _workspace(ws, need, dev):
    """The caller's workspace (a contiguous CUDA tensor; its size in bytes is passed on), or a
    fresh one of the size the library asks for."""
    if ws is None:
        return torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA tensor")
    return ws


def _nbytes(t):
    return t.numel() * t.element_size()


def _u8(t):
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def dsa_topk_workspace_bytes(T: int, L: int, k: int) -> int:
    return int(load().dsa_topk_workspace_bytes(T, L, k))


def dsa_prefill_workspace_bytes(T: int, L: int, H_I: int, H: int, k: int) -> int:
    return int(load().dsa_prefill_workspace_bytes(T, L, H_I, H, k))


def dsa_decode_workspace_bytes(B: int, max_len: int, total_tokens: int, H_I: int, H: int,
                               k: int) -> int:
    return int(load().dsa_decode_workspace_bytes(B, max_len, total_tokens, H_I, H, k))


def dsa_prefill_chunk_rows(T: int, L: int) -> int:
    return int(load().dsa_prefill_chunk_rows(T, L))


def dsa_index_scores(q8, q_scale, w, k8, k_scale, q_pos0: int, score_scale: float,
                     scores=None, write_masked: bool = True):
    """Lightning-indexer scores [T, L] (or into `scores` [T, ld >= L]); masked entries are
    -inf when write_masked, untouched otherwise."""
    lib = load()
    q8, k8 = _u8(q8), _u8(k8)
    T, H_I = q8.shape[0], q8.shape[1]
    L = k8.shape[0]
    _req(q8, torch.uint8, (T, H_I, 128), "q8")
    _req(q_scale, torch.float32, (T, H_I), "q_scale")
    _req(w, torch.float32, (T, H_I), "w")
    _req(k8, torch.uint8, (L, 128), "k8")
    _req(k_scale, torch.float32, (L,), "k_scale")
    if scores is None:
        scores = torch.empty((T, L), dtype=torch.float32, device=q8.device)
    _rows(scores, T, L, "scores")
    _check(lib.dsa_index_scores(_ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8), _ptr(k_scale), T, L,
                                H_I, q_pos0, score_scale, _ptr(scores), scores.stride(0),
                                int(bool(write_masked)), _stream()), "dsa_index_scores")
    return scores


def dsa_topk(scores, L: int, q_pos0: int, k: int, idx=None):
    """Per-row top-k of scores [T, >=L]: int32 [T, k], ascending positions, -1 padded."""
    lib = load()
    if not isinstance(scores, torch.Tensor) or scores.dim() != 2:
        raise ValueError("scores must be float32 [T, >=L] with unit column stride")
    T = scores.shape[0]
    _rows(scores, T, L, "scores")
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    _req(idx, torch.int32, (T, k), "idx")
    _check(lib.dsa_topk(_ptr(scores), scores.stride(0), T, L, q_pos0, k, _ptr(idx), None, 0,
                        _stream()), "dsa_topk")
    return idx


def dsa_sparse_mla(q, kv, idx, sm_scale: float, out=None, lse=None):
    """Attention of q [T,H,576] over the kv rows listed in idx [T,k]: (out, lse)."""
    lib = load()
    T, H = q.shape[0], q.shape[1]
    L, k = kv.shape[0], idx.shape[1]
    _req(q, torch.bfloat16, (T, H, 576), "q")
    _req(kv, torch.bfloat16, (L, 576), "kv")
    _req(idx, torch.int32, (T, k), "idx")
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _req(out, torch.bfloat16, (T, H, 512), "out")
    _req(lse, torch.float32, (T, H), "lse")
    _check(lib.dsa_sparse_mla(_ptr(q), _ptr(kv), _ptr(idx), T, L, H, k, sm_scale, _ptr(out),
                              _ptr(lse), _stream()), "dsa_sparse_mla")
    return out, lse


def dsa_prefill(q8, q_scale, w, k8, k_scale, q, kv, k: int, q_pos0: int, score_scale: float,
                sm_scale: float, out=None, lse=None, idx_out=None, workspace=None):
    """Whole prefill path (indexer -> top-k -> sparse MLA): (out, lse, idx_out)."""
    lib = load()
    q8, k8 = _u8(q8), _u8(k8)
    T, H_I = q8.shape[0], q8.shape[1]
    L, H = k8.shape[0], q.shape[1]
    _req(q8, torch.uint8, (T, H_I, 128), "q8")
    _req(q_scale, torch.float32, (T, H_I), "q_scale")
    _req(w, torch.float32, (T, H_I), "w")
    _req(k8, torch.uint8, (L, 128), "k8")
    _req(k_scale, torch.float32, (L,), "k_scale")
    _req(q, torch.bfloat16, (T, H, 576), "q")
    _req(kv, torch.bfloat16, (L, 576), "kv")
    dev = q.device
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _req(out, torch.bfloat16, (T, H, 512), "out")
    _req(lse, torch.float32, (T, H), "lse")
    if idx_out is not None:
        _req(idx_out, torch.int32, (T, k), "idx_out")
    need = dsa_prefill_workspace_bytes(T, L, H_I, H, k)
    workspace = _workspace(workspace, need, dev)
    _check(lib.dsa_prefill(_ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(q),
                           _ptr(kv), T, L, H_I, H, k, q_pos0, score_scale, sm_scale, _ptr(out),
                           _ptr(lse), _ptr(idx_out), _ptr(workspace), _nbytes(workspace),
                           _stream()), "dsa_prefill")
    return out, lse, idx_out


def _host_cu(cu, name):
    """cu_seqlens as a contiguous host int64 array (they size the launches)."""
    t = torch.as_tensor(cu, dtype=torch.int64)
    if t.is_cuda or t.dim() != 1 or t.numel() < 1:
        raise TypeError("%s must be a host int64 vector [B+1]" % name)
    return t.contiguous()


def dsa_prefill_varlen_workspace_bytes(cu_seqlens_q, cu_seqlens_k, H_I: int, H: int,
                                       k: int) -> int:
    cq, ck = _host_cu(cu_seqlens_q, "cu_seqlens_q"), _host_cu(cu_seqlens_k, "cu_seqlens_k")
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    return int(load().dsa_prefill_varlen_workspace_bytes(cq.numel() - 1, _ptr(cq), _ptr(ck),
                                                         H_I, H, k))


def dsa_prefill_varlen(cu_seqlens_q, cu_seqlens_k, q8, q_scale, w, k8, k_scale, q, kv, k: int,
                       score_scale: float, sm_scale: float, out=None, lse=None, idx_out=None,
                       workspace=None):
    """Packed prefill of B sequences (host cu_seqlens [B+1]); sequence b's queries are its
    last T_b tokens.  Returns (out [Tq,H,512], lse [Tq,H], idx_out)."""
    lib = load()
    cq, ck = _host_cu(cu_seqlens_q, "cu_seqlens_q"), _host_cu(cu_seqlens_k, "cu_seqlens_k")
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    B = cq.numel() - 1
    q8, k8 = _u8(q8), _u8(k8)
    Tq, H_I = q8.shape[0], q8.shape[1]
    Lk, H = k8.shape[0], q.shape[1]
    if int(cq[-1]) != Tq or int(ck[-1]) != Lk:
        raise ValueError("cu_seqlens must end at the packed row counts (%d, %d)" % (Tq, Lk))
    _req(q8, torch.uint8, (Tq, H_I, 128), "q8")
    _req(q_scale, torch.float32, (Tq, H_I), "q_scale")
    _req(w, torch.float32, (Tq, H_I), "w")
    _req(k8, torch.uint8, (Lk, 128), "k8")
    _req(k_scale, torch.float32, (Lk,), "k_scale")
    _req(q, torch.bfloat16, (Tq, H, 576), "q")
    _req(kv, torch.bfloat16, (Lk, 576), "kv")
    dev = q.device
    if out is None:
        out = torch.empty((Tq, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    _req(out, torch.bfloat16, (Tq, H, 512), "out")
    _req(lse, torch.float32, (Tq, H), "lse")
    if idx_out is not None:
        _req(idx_out, torch.int32, (Tq, k), "idx_out")
    need = int(lib.dsa_prefill_varlen_workspace_bytes(B, _ptr(cq), _ptr(ck), H_I, H, k))
    workspace = _workspace(workspace, need, dev)
    _check(lib.dsa_prefill_varlen(B, _ptr(cq), _ptr(ck), _ptr(q8), _ptr(q_scale), _ptr(w),
                                  _ptr(k8), _ptr(k_scale), _ptr(q), _ptr(kv), H_I, H, k,
                                  score_scale, sm_scale, _ptr(out), _ptr(lse), _ptr(idx_out),
                                  _ptr(workspace), _nbytes(workspace), _stream()),
           "dsa_prefill_varlen")
    return out, lse, idx_out


def dsa_attention_lse(q, kv, q_pos0: int, sm_scale: float, lse=None):
    """Per-head log-sum-exp [T, H] of dense causal attention of q [T,H,576] over kv [L,576]."""
    lib = load()
    T, H, L = q.shape[0], q.shape[1], kv.shape[0]
    _req(q, torch.bfloat16, (T, H, 576), "q")
    _req(kv, torch.bfloat16, (L, 576), "kv")
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _req(lse, torch.float32, (T, H), "lse")
    _check(lib.dsa_attention_lse(_ptr(q), _ptr(kv), T, L, H, q_pos0, sm_scale, _ptr(lse),
                                 _stream()), "dsa_attention_lse")
    return lse


def dsa_attention_distribution(q, kv, lse, q_pos0: int, sm_scale: float, P=None):
    """Head-averaged dense attention distribution P [T, >=L] (entries past each row's
    position are left as they were)."""
    lib = load()
    T, H, L = q.shape[0], q.shape[1], kv.shape[0]
    _req(q, torch.bfloat16, (T, H, 576), "q")
    _req(kv, torch.bfloat16, (L, 576), "kv")
    _req(lse, torch.float32, (T, H), "lse")
    if P is None:
        P = torch.zeros((T, L), dtype=torch.float32, device=q.device)
    _rows(P, T, L, "P")
    _check(lib.dsa_attention_distribution(_ptr(q), _ptr(kv), _ptr(lse), T, L, H, q_pos0,
                                          sm_scale, _ptr(P), P.stride(0), _stream()),
           "dsa_attention_distribution")
    return P


def dsa_indexer_warmup_workspace_bytes(T: int, L: int, H_I: int, H: int) -> int:
    return int(load().dsa_indexer_warmup_workspace_bytes(T, L, H_I, H))


def dsa_indexer_warmup(q8, q_scale, w, k8, k_scale, q, kv, q_pos0: int, score_scale: float,
                       sm_scale: float, out=None, workspace=None):
    """Indexer warm-up loss and gradient: dict of kl [T], dq [T,H_I,128], dw [T,H_I],
    dk [L,128], lse_teacher [T,H], lse_index [T] (float32; `out` may supply any of them)."""
    lib = load()
    q8, k8 = _u8(q8), _u8(k8)
    T, H_I = q8.shape[0], q8.shape[1]
    L, H = k8.shape[0], q.shape[1]
    _req(q8, torch.uint8, (T, H_I, 128), "q8")
    _req(q_scale, torch.float32, (T, H_I), "q_scale")
    _req(w, torch.float32, (T, H_I), "w")
    _req(k8, torch.uint8, (L, 128), "k8")
    _req(k_scale, torch.float32, (L,), "k_scale")
    _req(q, torch.bfloat16, (T, H, 576), "q")
    _req(kv, torch.bfloat16, (L, 576), "kv")
    dev = q.device
    shapes = dict(kl=(T,), dq=(T, H_I, 128), dw=(T, H_I), dk=(L, 128), lse_teacher=(T, H),
                  lse_index=(T,))
    res = dict(out or {})
    for key, shp in shapes.items():
        if key not in res:
            res[key] = torch.empty(shp, dtype=torch.float32, device=dev)
        _req(res[key], torch.float32, shp, key)
    need = dsa_indexer_warmup_workspace_bytes(T, L, H_I, H)
    workspace = _workspace(workspace, need, dev)
    _check(lib.dsa_indexer_warmup(_ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8), _ptr(k_scale),
                                  _ptr(q), _ptr(kv), T, L, H_I, H, q_pos0, score_scale, sm_scale,
                                  _ptr(res["kl"]), _ptr(res["dq"]), _ptr(res["dw"]),
                                  _ptr(res["dk"]), _ptr(res["lse_teacher"]),
                                  _ptr(res["lse_index"]), _ptr(workspace), _nbytes(workspace),
                                  _stream()), "dsa_indexer_warmup")
    return res


def dsa_decode(seq_start, max_len: int, q8, q_scale, w, k8, k_scale, q, kv, k: int,
               score_scale: float, sm_scale: float, out=None, lse=None, idx_out=None,
               workspace=None):
    """One decode step over B packed sequences: (out [B,H,512], lse [B,H], idx_out)."""
    lib = load()
    q8, k8 = _u8(q8), _u8(k8)
    B, H_I = q8.shape[0], q8.shape[1]
    N, H = k8.shape[0], q.shape[1]
    _req(seq_start, torch.int64, (B + 1,), "seq_start")
    _req(q8, torch.uint8, (B, H_I, 128), "q8")
    _req(q_scale, torch.float32, (B, H_I), "q_scale")
    _req(w, torch.float32, (B, H_I), "w")
    _req(k8, torch.uint8, (N, 128), "k8")
    _req(k_scale, torch.float32, (N,), "k_scale")
    _req(q, torch.bfloat16, (B, H, 576), "q")
    _req(kv, torch.bfloat16, (N, 576), "kv")
    dev = q.device
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _req(out, torch.bfloat16, (B, H, 512), "out")
    _req(lse, torch.float32, (B, H), "lse")
    if idx_out is not None:
        _req(idx_out, torch.int32, (B, k), "idx_out")
    need = dsa_decode_workspace_bytes(B, max_len, N, H_I, H, k)
    workspace = _workspace(workspace, need, dev)
    _check(lib.dsa_decode(B, _ptr(seq_start), max_len, N, _ptr(q8), _ptr(q_scale), _ptr(w),
                          _ptr(k8), _ptr(k_scale), _ptr(q), _ptr(kv), H_I, H, k, score_scale,
                          sm_scale, _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(workspace),
                          _nbytes(workspace), _stream()), "dsa_decode")
    return out, lse, idx_out


def dsa_decode_noalloc_scratch_bytes() -> int:
    return int(load().dsa_decode_noalloc_scratch_bytes())


def dsa_decode_noalloc(seq_start, max_len: int, q8, q_scale, w, k8, k_scale, q, kv, k: int,
                       score_scale: float, sm_scale: float, out=None, lse=None, idx_out=None):
    """dsa_decode on the library's fixed per-GPU scratch array instead of a workspace (for
    callers that cannot allocate; pass `out`, `lse` and `idx_out` to allocate nothing here
    either).  Calls that overlap on one GPU race on that array."""
    lib = load()
    q8, k8 = _u8(q8), _u8(k8)
    B, H_I = q8.shape[0], q8.shape[1]
    N, H = k8.shape[0], q.shape[1]
    _req(seq_start, torch.int64, (B + 1,), "seq_start")
    _req(q8, torch.uint8, (B, H_I, 128), "q8")
    _req(q_scale, torch.float32, (B, H_I), "q_scale")
    _req(w, torch.float32, (B, H_I), "w")
    _req(k8, torch.uint8, (N, 128), "k8")
    _req(k_scale, torch.float32, (N,), "k_scale")
    _req(q, torch.bfloat16, (B, H, 576), "q")
    _req(kv, torch.bfloat16, (N, 576), "kv")
    dev = q.device
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _req(out, torch.bfloat16, (B, H, 512), "out")
    _req(lse, torch.float32, (B, H), "lse")
    if idx_out is not None:
        _req(idx_out, torch.int32, (B, k), "idx_out")
    _check(lib.dsa_decode_noalloc(B, _ptr(seq_start), max_len, N, _ptr(q8), _ptr(q_scale),
                                  _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(q), _ptr(kv), H_I, H, k,
                                  score_scale, sm_scale, _ptr(out), _ptr(lse), _ptr(idx_out),
                                  _stream()), "dsa_decode_noalloc")
    return out, lse, idx_out


def dsa_quantize_fp8(x, q8=None, scale=None):
    """Per-128-vector e4m3fn quantisation of x [..., 128] (float32 or bfloat16):
    (q8 uint8 [..., 128], scale float32 [...])."""
    lib = load()
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype not in (torch.float32,
                                                                            torch.bfloat16):
        raise TypeError("x must be a float32 or bfloat16 CUDA tensor")
    if x.shape[-1] != 128 or not x.is_contiguous():
        raise ValueError("x must be contiguous [..., 128]")
    lead = tuple(x.shape[:-1])
    n = x.numel() // 128
    if q8 is None:
        q8 = torch.empty(lead + (128,), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(lead, dtype=torch.float32, device=x.device)
    _req(q8, torch.uint8, lead + (128,), "q8")
    _req(scale, torch.float32, lead, "scale")
    _check(lib.dsa_quantize_fp8(_ptr(x), int(x.dtype == torch.bfloat16), n, _ptr(q8),
                                _ptr(scale), _stream()), "dsa_quantize_fp8")
    return q8, scale


def dsa_decode_append(seq_start, k_new, kv_new, k8_cache, k_scale_cache, kv_cache):
    """Write each sequence's new token into row seq_start[b+1]-1 of the packed caches
    (in place): k_new [B,128] float32/bfloat16, kv_new [B,576] bfloat16."""
    lib = load()
    B = k_new.shape[0]
    N = kv_cache.shape[0]
    _req(seq_start, torch.int64, (B + 1,), "seq_start")
    if not isinstance(k_new, torch.Tensor) or not k_new.is_cuda or k_new.dtype not in (
            torch.float32, torch.bfloat16):
        raise TypeError("k_new must be a float32 or bfloat16 CUDA tensor")
    if tuple(k_new.shape) != (B, 128) or not k_new.is_contiguous():
        raise ValueError("k_new must be contiguous [B, 128]")
    _req(kv_new, torch.bfloat16, (B, 576), "kv_new")
    k8_cache = _u8(k8_cache)
    _req(k8_cache, torch.uint8, (N, 128), "k8_cache")
    _req(k_scale_cache, torch.float32, (N,), "k_scale_cache")
    _req(kv_cache, torch.bfloat16, (N, 576), "kv_cache")
    _check(lib.dsa_decode_append(B, _ptr(seq_start), _ptr(k_new),
                                 int(k_new.dtype == torch.bfloat16), _ptr(kv_new),
                                 _ptr(k8_cache), _ptr(k_scale_cache), _ptr(kv_cache),
                                 _stream()), "dsa_decode_append")
    return k8_cache, k_scale_cache, kv_cache


def dsa_window_indices(T: int, L: int, q_pos0: int, window: int, idx=None, device="cuda"):
    """Sliding-window index lists int32 [T, window]: max(0, p-window+1) .. p, -1 padded."""
    lib = load()
    if idx is None:
        idx = torch.empty((T, window), dtype=torch.int32, device=device)
    _req(idx, torch.int32, (T, window), "idx")
    _check(lib.dsa_window_indices(T, L, q_pos0, window, _ptr(idx), _stream()),
           "dsa_window_indices")
    return idx


def dsa_local_selected_indices(sel, L: int, q_pos0: int, window: int, out=None):
    """Ascending union of each row's window and its selected positions sel [T, k] (ascending,
    as dsa_topk writes them): int32 [T, window + k], -1 padded."""
    lib = load()
    T, k = sel.shape
    _req(sel, torch.int32, (T, k), "sel")
    if out is None:
        out = torch.empty((T, window + k), dtype=torch.int32, device=sel.device)
    _req(out, torch.int32, (T, window + k), "out")
    _check(lib.dsa_local_selected_indices(_ptr(sel), T, L, q_pos0, k, window, _ptr(out),
                                          _stream()), "dsa_local_selected_indices")
    return out
