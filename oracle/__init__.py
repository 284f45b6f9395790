"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It wraps ``oracle.c`` (plain C, fp64, exact int64 indexer dots,
built with gcc and OpenMP) with numpy marshalling, and composes the per-step functions
into the prefill and decode paths.  It shares no code with the HIP library and never
imports it.

Pins (what fixes this oracle besides itself) live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (OpenMP).  Returns its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
            lib.ora_e4m3fn_value.restype = dbl
            lib.ora_e4m3fn_value.argtypes = [ctypes.c_uint8]
            lib.ora_bf16_value.restype = dbl
            lib.ora_bf16_value.argtypes = [ctypes.c_uint16]
            lib.ora_index_scores.argtypes = [P, P, P, P, P, i64, i32, i64, dbl, P, i64, P, P]
            lib.ora_topk_sort.argtypes = [P, i64, i64, P, i32, P]
            lib.ora_topk_select.argtypes = [P, i64, i64, P, i32, P]
            lib.ora_sparse_mla.argtypes = [P, P, P, i64, i32, i32, dbl, P, i64, P, P]
            lib.ora_dense_mla.argtypes = [P, P, i64, i32, i64, dbl, P, i64, P, P]
            lib.ora_quantize_e4m3.argtypes = [P, i32, i64, P, P]
            lib.ora_decode_append.argtypes = [i32, P, P, i32, P, P, P, P]
            lib.ora_window_indices.argtypes = [i64, i64, i32, P]
            lib.ora_local_selected.argtypes = [P, i64, i32, i64, i32, P]
            lib.ora_warmup.argtypes = [P, P, P, P, i64, P, P, i64, i32, i32, dbl, dbl] + [P] * 14
            lib.ora_num_threads.restype = i32
            _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _rows(rows, T):
    if rows is None:
        return np.arange(T, dtype=np.int64)
    return _c(rows, np.int64)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle: invalid input to %s" % what)


def num_threads() -> int:
    return int(_load().ora_num_threads())


def e4m3fn_values(codes) -> np.ndarray:
    lib = _load()
    return np.array([lib.ora_e4m3fn_value(int(c)) for c in np.ravel(codes)], dtype=np.float64)


def bf16_values(bits) -> np.ndarray:
    lib = _load()
    return np.array([lib.ora_bf16_value(int(b)) for b in np.ravel(bits)], dtype=np.float64)


_TABLES = {}


def _decode_tables():
    """fp64 value of every e4m3fn code and every bf16 bit pattern (the pinned decoders)."""
    if not _TABLES:
        _TABLES["e4m3"] = e4m3fn_values(np.arange(256))
        _TABLES["bf16"] = bf16_values(np.arange(65536))
    return _TABLES["e4m3"], _TABLES["bf16"]


def warmup_inputs(inp: dict, rows=None):
    """Real-valued (fp64) warm-up inputs from the stored formats: the indexer's dequantised
    query and key vectors QI = qs * q8, KI = ks * k8, the weights w, and the MLA query and
    cache rows, for the given query rows (positions q_pos0 + row)."""
    e4, b16 = _decode_tables()
    T = inp["q8"].shape[0]
    r = _rows(rows, T)
    q8, qs = np.asarray(inp["q8"])[r], np.asarray(inp["qs"], np.float64)[r]
    return dict(QI=e4[q8] * qs[..., None], w=np.asarray(inp["w"], np.float64)[r],
                q=b16[np.asarray(inp["q"])[r]], pos=inp["q_pos0"] + r,
                KI=e4[np.asarray(inp["k8"])] * np.asarray(inp["ks"], np.float64)[:, None],
                kv=b16[np.asarray(inp["kv"])], c=float(inp["score_scale"]),
                sm_scale=float(inp["sm_scale"]))


def warmup(x: dict, want_dk=False, bounds=False, dist=False):
    """Indexer warm-up loss and gradient on real-valued inputs (see warmup_inputs): per row
    kl, teacher lse_t [., H], student lse_i, dq [., H_I, 128], dw [., H_I]; with want_dk the
    key gradient dk [L, 128] summed over the given rows; with dist the target P and the score
    gradient G [., L]; with bounds the magnitude sums the tolerances are built from."""
    QI, w, q, KI, kv = (_c(x[k], np.float64) for k in ("QI", "w", "q", "KI", "kv"))
    pos = _c(x["pos"], np.int64)
    n, H_I = QI.shape[0], QI.shape[1]
    H, L = q.shape[1], KI.shape[0]
    assert QI.shape[2] == 128 and q.shape == (n, H, 576) and kv.shape == (L, 576)
    out = dict(kl=np.empty(n), lse_t=np.empty((n, H)), lse_i=np.empty(n),
               dq=np.empty((n, H_I, 128)), dw=np.empty((n, H_I)))
    opt = {}
    if dist:
        opt["P"], opt["G"] = np.empty((n, L)), np.empty((n, L))
    if want_dk:
        opt["dk"] = np.empty((L, 128))
    if bounds:
        opt.update(kl_bnd=np.empty(n), dw_bnd=np.empty((n, H_I)), dq_bnd=np.empty((n, H_I, 128)),
                   dq_amb=np.empty((n, H_I, 128)))
        if want_dk:
            opt.update(dk_bnd=np.empty((L, 128)), dk_amb=np.empty((L, 128)))
    out.update(opt)
    ptr = lambda k: _p(out[k]) if k in out else None
    rc = _load().ora_warmup(_p(QI), _p(w), _p(q), _p(pos), n, _p(KI), _p(kv), L, H_I, H,
                            x["c"], x["sm_scale"], ptr("kl"), ptr("lse_t"), ptr("lse_i"),
                            ptr("dq"), ptr("dw"), ptr("P"), ptr("G"), ptr("dk"), ptr("kl_bnd"),
                            ptr("dw_bnd"), ptr("dq_bnd"), ptr("dq_amb"), ptr("dk_bnd"),
                            ptr("dk_amb"))
    _check(rc, "warmup")
    return out


def quantize_e4m3(x):
    """Per-128-vector e4m3fn quantisation: x [..., 128] float32, or uint16 bf16 bits ->
    (codes uint8 [..., 128], scales float32 [...])."""
    x = np.asarray(x)
    bf16 = x.dtype == np.uint16
    x = _c(x, np.uint16 if bf16 else np.float32)
    assert x.shape[-1] == 128
    n = x.size // 128
    q8 = np.empty(x.shape, np.uint8)
    sc = np.empty(x.shape[:-1], np.float32)
    _check(_load().ora_quantize_e4m3(_p(x), int(bf16), n, _p(q8), _p(sc)), "quantize_e4m3")
    return q8, sc


def decode_append(seq_start, k_new, kv_new, k8_cache, ks_cache, kv_cache):
    """Write each sequence's new token into row seq_start[b+1]-1 of the caches (in place);
    k_new [B,128] float32 or uint16 bf16 bits, kv_new [B,576] uint16."""
    st = _c(seq_start, np.int64)
    k_new = np.asarray(k_new)
    bf16 = k_new.dtype == np.uint16
    k_new = _c(k_new, np.uint16 if bf16 else np.float32)
    kv_new = _c(kv_new, np.uint16)
    for a, dt in ((k8_cache, np.uint8), (ks_cache, np.float32), (kv_cache, np.uint16)):
        assert a.dtype == dt and a.flags["C_CONTIGUOUS"]
    B = len(st) - 1
    _check(_load().ora_decode_append(B, _p(st), _p(k_new), int(bf16), _p(kv_new), _p(k8_cache),
                                     _p(ks_cache), _p(kv_cache)), "decode_append")


def window_indices(T: int, q_pos0: int, W: int):
    """int32 [T, W]: positions max(0, p-W+1) .. p of each row, ascending, -1 padded."""
    out = np.empty((T, W), np.int32)
    _check(_load().ora_window_indices(T, q_pos0, W, _p(out)), "window_indices")
    return out


def local_selected(sel, q_pos0: int, W: int):
    """int32 [T, W + k]: ascending union of each row's window and its selected positions."""
    sel = _c(sel, np.int32)
    T, k = sel.shape
    out = np.empty((T, W + k), np.int32)
    _check(_load().ora_local_selected(_p(sel), T, k, q_pos0, W, _p(out)), "local_selected")
    return out


def index_scores(q8, qs, w, k8, ks, q_pos0: int, c: float, rows=None, with_bound=False):
    """fp64 scores [n_rows, L] (and the conditioning bound) of the lightning indexer."""
    q8, k8 = _c(q8, np.uint8), _c(k8, np.uint8)
    qs, w, ks = _c(qs, np.float32), _c(w, np.float32), _c(ks, np.float32)
    T, H_I = q8.shape[0], q8.shape[1]
    L = k8.shape[0]
    assert q8.shape[2] == 128 and k8.shape[1] == 128 and qs.shape == (T, H_I) == w.shape
    r = _rows(rows, T)
    scores = np.empty((len(r), L), np.float64)
    bound = np.empty((len(r), L), np.float64) if with_bound else None
    rc = _load().ora_index_scores(_p(q8), _p(qs), _p(w), _p(k8), _p(ks), L, H_I, q_pos0, c,
                                  _p(r), len(r), _p(scores),
                                  _p(bound) if with_bound else None)
    _check(rc, "index_scores")
    return (scores, bound) if with_bound else scores


def topk(scores, n_vis, k: int, method: str = "sort"):
    """int32 [n_rows, k]: ascending selected positions, -1 padded."""
    s = _c(scores, np.float64)
    n = _c(n_vis, np.int64)
    assert s.ndim == 2 and n.shape == (s.shape[0],)
    idx = np.empty((s.shape[0], k), np.int32)
    fn = {"sort": _load().ora_topk_sort, "select": _load().ora_topk_select}[method]
    _check(fn(_p(s), s.shape[1], s.shape[0], _p(n), k, _p(idx)), "topk")
    return idx


def sparse_mla(q, kv, idx, sm_scale: float, rows=None):
    """fp64 (out [n_rows, H, 512], lse [n_rows, H]) of attention over idx's rows."""
    q, kv, idx = _c(q, np.uint16), _c(kv, np.uint16), _c(idx, np.int32)
    T, H = q.shape[0], q.shape[1]
    L, k = kv.shape[0], idx.shape[1]
    assert q.shape[2] == 576 and kv.shape[1] == 576 and idx.shape[0] == T
    r = _rows(rows, T)
    out = np.empty((len(r), H, 512), np.float64)
    lse = np.empty((len(r), H), np.float64)
    _check(_load().ora_sparse_mla(_p(q), _p(kv), _p(idx), L, H, k, sm_scale, _p(r), len(r),
                                  _p(out), _p(lse)), "sparse_mla")
    return out, lse


def dense_mla(q, kv, q_pos0: int, sm_scale: float, rows=None):
    """fp64 (out, lse) of causal attention over every visible token."""
    q, kv = _c(q, np.uint16), _c(kv, np.uint16)
    T, H = q.shape[0], q.shape[1]
    L = kv.shape[0]
    r = _rows(rows, T)
    out = np.empty((len(r), H, 512), np.float64)
    lse = np.empty((len(r), H), np.float64)
    _check(_load().ora_dense_mla(_p(q), _p(kv), L, H, q_pos0, sm_scale, _p(r), len(r),
                                 _p(out), _p(lse)), "dense_mla")
    return out, lse


def prefill(inp: dict, rows=None, with_bound=False):
    """Whole prefill path on host arrays (see synth.host_arrays) for the given query rows:
    indexer scores -> top-k -> sparse MLA.  Rows that see <= k tokens select all of them
    without consulting the scores."""
    T, L, k = inp["T"], inp["L"], inp["k"]
    r = _rows(rows, T)
    res = index_scores(inp["q8"], inp["qs"], inp["w"], inp["k8"], inp["ks"], inp["q_pos0"],
                       inp["score_scale"], rows=r, with_bound=with_bound)
    scores, bound = res if with_bound else (res, None)
    n_vis = inp["q_pos0"] + r + 1
    idx = topk(scores, n_vis, k)
    full_idx = np.full((T, k), -1, np.int32)
    full_idx[r] = idx
    out, lse = sparse_mla(inp["q"], inp["kv"], full_idx, inp["sm_scale"], rows=r)
    return dict(rows=r, scores=scores, bound=bound, n_vis=n_vis, idx=idx, out=out, lse=lse)


def prefill_varlen(inp: dict, seqs=None, with_bound=False):
    """Packed prefill of B sequences on host arrays (see synth.make_varlen): sequence b owns
    query rows [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]); its T_b queries are
    its last T_b tokens, so row t of it sits at position L_b - T_b + t and sees that
    sequence's tokens 0 .. L_b - T_b + t only.  Each sequence is one prefill call on its own
    slices; returns one prefill() result per requested sequence (indices are positions within
    the sequence)."""
    cu_q = np.asarray(inp["cu_q"], np.int64)
    cu_k = np.asarray(inp["cu_k"], np.int64)
    seqs = range(len(cu_q) - 1) if seqs is None else seqs
    res = []
    for b in seqs:
        qa, qe, ka, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        T, L = qe - qa, ke - ka
        if T == 0:
            res.append(None)
            continue
        one = dict(T=T, L=L, k=inp["k"], q_pos0=L - T, score_scale=inp["score_scale"],
                   sm_scale=inp["sm_scale"])
        for key in ("q8", "qs", "w", "q"):
            one[key] = inp[key][qa:qe]
        for key in ("k8", "ks", "kv"):
            one[key] = inp[key][ka:ke]
        r = prefill(one, with_bound=with_bound)
        r.update(seq=int(b), T=T, L=L, q_pos0=L - T)
        res.append(r)
    return res


def decode(inp: dict, seqs=None, with_bound=False):
    """Decode step on host arrays: sequence b owns cache rows [seq_start[b], seq_start[b+1])
    and its one query sits at position L_b - 1 (it sees its whole cache, itself included)."""
    st = np.asarray(inp["seq_start"], np.int64)
    B, k = inp["B"], inp["k"]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    res = []
    for b in seqs:
        a, e = int(st[b]), int(st[b + 1])
        Lb = e - a
        one = lambda x: x[b:b + 1]
        sc = index_scores(one(inp["q8"]), one(inp["qs"]), one(inp["w"]), inp["k8"][a:e],
                          inp["ks"][a:e], Lb - 1, inp["score_scale"], with_bound=with_bound)
        sc, bd = sc if with_bound else (sc, None)
        idx = topk(sc, np.array([Lb]), k)
        out, lse = sparse_mla(one(inp["q"]), inp["kv"][a:e], idx, inp["sm_scale"])
        res.append(dict(seq=int(b), L=Lb, scores=sc[0], bound=None if bd is None else bd[0],
                        idx=idx[0], out=out[0], lse=lse[0]))
    return res
