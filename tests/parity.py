"""Parity rules between the HIP path and the CPU oracle (test infrastructure).

* indexer scores: |g - o| <= 1e-3 |o| + 2^-16 A[t,s], A the conditioning bound
  ks * sum_h |a'_h| sum_d |q k| (covers fp32 cancellation between signed heads, about
  1.3x the worst-case fp32 summation error (128 + 64) 2^-24); masked entries exactly -inf.
* top-k on the GPU's own fp32 scores: exactly the oracle's selection of the same values.
* end-to-end indices: same count min(k, n_t); every position in the symmetric difference
  has an oracle score within tol(tau) of the oracle's k-th score tau (a near-tie).
* sparse MLA, against the oracle run on the GPU's own indices: |out_g - out_o| <= 1e-2 +
  2^-8 |out_o| per element (1e-2 for O(1) outputs plus the round-to-nearest bf16 rounding of
  the output itself: bf16 keeps 8 significant bits, so an output of magnitude 2..4, which
  rows averaging only a few latent rows produce, cannot be stored closer than 2^-8 |o|),
  per (row, head) ||delta||_2 / ||o||_2 <= 1e-2, |delta lse| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

SCORE_RTOL = 1e-3
SCORE_FLOOR = 2.0 ** -16
OUT_ATOL = 1e-2
OUT_BF16_REL = 2.0 ** -8
OUT_REL_L2 = 1e-2
LSE_ATOL = 1e-3


def to_device(inp: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check_scores(g: np.ndarray, o: np.ndarray, bound: np.ndarray, what=""):
    g = np.asarray(g, np.float64)
    masked = np.isneginf(o)
    assert np.array_equal(np.isneginf(g), masked), "%s: mask pattern differs" % what
    vis = ~masked
    err = np.abs(g[vis] - o[vis])
    tol = SCORE_RTOL * np.abs(o[vis]) + SCORE_FLOOR * bound[vis]
    bad = err > tol
    assert not bad.any(), "%s: %d scores out of tolerance, worst err %.3g (tol %.3g)" % (
        what, bad.sum(), err[bad].max(), tol[bad][np.argmax(err[bad])])
    return float(err.max(initial=0.0))


def check_topk_exact(gpu_idx: np.ndarray, gpu_scores: np.ndarray, n_vis, k: int, what=""):
    want = oracle.topk(np.asarray(gpu_scores, np.float64), n_vis, k)
    got = np.asarray(gpu_idx)
    if not np.array_equal(got, want):
        r = np.nonzero((got != want).any(1))[0]
        raise AssertionError("%s: top-k differs on %d rows, first %d: got %s want %s" % (
            what, len(r), r[0], got[r[0]][:16], want[r[0]][:16]))


def check_indices_near_ties(gpu_idx, ora_idx, ora_scores, bound, n_vis, k: int, what=""):
    """Returns the number of near-tie swaps; fails on any other difference."""
    swaps = 0
    for r in range(len(n_vis)):
        n = int(n_vis[r])
        g = np.asarray(gpu_idx[r])
        o = np.asarray(ora_idx[r])
        gs, os_ = set(g[g >= 0].tolist()), set(o[o >= 0].tolist())
        assert len(gs) == len(os_) == min(n, k), "%s row %d: wrong count" % (what, r)
        assert len(set(g[g >= 0].tolist())) == (g >= 0).sum(), "%s row %d: duplicates" % (what, r)
        assert all(0 <= s < n for s in gs), "%s row %d: index outside the visible range" % (what, r)
        diff = gs ^ os_
        if not diff:
            continue
        row = ora_scores[r, :n]
        tau = np.sort(row)[::-1][k - 1]
        tol = SCORE_RTOL * abs(tau) + SCORE_FLOOR * bound[r, :n].max()
        for s in diff:
            assert abs(row[s] - tau) <= tol, "%s row %d: position %d (score %.9g) is not a " \
                "near-tie of tau %.9g (tol %.3g)" % (what, r, s, row[s], tau, tol)
        swaps += len(diff) // 2
    return swaps


def check_mla(out_g: np.ndarray, lse_g: np.ndarray, out_o: np.ndarray, lse_o: np.ndarray,
              what=""):
    d = np.abs(out_g - out_o)
    lim = OUT_ATOL + OUT_BF16_REL * np.abs(out_o)
    assert np.all(d <= lim), "%s: |dout| %.3g exceeds 1e-2 + 2^-8|o| (|o| = %.3g)" % (
        what, d.max(), np.abs(out_o).ravel()[np.argmax((d - lim).ravel())])
    num = np.sqrt(((out_g - out_o) ** 2).sum(-1))
    den = np.sqrt((out_o ** 2).sum(-1))
    rel = num / np.maximum(den, 1e-30)
    assert rel.max(initial=0.0) <= OUT_REL_L2, "%s: rel L2 %.3g" % (what, rel.max())
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lse_g), fin), "%s: lse finiteness differs" % what
    dl = np.abs(lse_g[fin] - lse_o[fin])
    assert dl.max(initial=0.0) <= LSE_ATOL, "%s: max |dlse| %.3g" % (what, dl.max())
    return float(d.max(initial=0.0)), float(rel.max(initial=0.0)), float(dl.max(initial=0.0))


# ------------------------------------------------------------------------- reporting
# Per-config parity statistics (near-tie swaps, planted-token recall, worst errors), printed
# in pytest's terminal summary and, when DSA_PARITY_REPORT names a file, written there as JSON.
REPORT: dict = {}


def report(config: str, **stats):
    REPORT.setdefault(config, {}).update(stats)


def _np(t):
    return t.detach().cpu().numpy()


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_prefill_rows(d: dict, rows, k):
    """Oracle scores, bound and selection of selected rows of a device prefill workload, as
    one dict per row (all rows in one oracle call: see oracle_rows)."""
    h = dict(q8=_np(d["q8"]), qs=_np(d["qs"]), w=_np(d["w"]), k8=_np(d["k8"]), ks=_np(d["ks"]),
             q_pos0=d["q_pos0"], score_scale=d["score_scale"])
    o = oracle_rows(h, rows, k)
    return [dict(t=int(t), n=int(o["n_vis"][i]), scores=o["scores"][i], bound=o["bound"][i],
                 idx=o["idx"][i]) for i, t in enumerate(o["rows"])]


def oracle_rows(h: dict, rows, k: int) -> dict:
    """Oracle indexer scores (with their conditioning bound) and top-k selection of the given
    query rows of a prefill workload (host arrays q8, qs, w, k8, ks and the scalars), in one
    call per step so that the oracle's OpenMP loop spreads the rows over the host cores."""
    r = np.asarray(rows, np.int64)
    sc, bd = oracle.index_scores(h["q8"], h["qs"], h["w"], h["k8"], h["ks"], h["q_pos0"],
                                 h["score_scale"], rows=r, with_bound=True)
    n_vis = h["q_pos0"] + r + 1
    return dict(rows=r, scores=sc, bound=bd, n_vis=n_vis, idx=oracle.topk(sc, n_vis, k))


def host_prefill(d: dict, q_rows=None) -> dict:
    """Host copies of a device prefill workload's indexer inputs and cache (and, if q_rows is
    given, of those rows of the MLA query only)."""
    h = dict(q8=_np(d["q8"]), qs=_np(d["qs"]), w=_np(d["w"]), k8=_np(d["k8"]), ks=_np(d["ks"]),
             kv=_u16(d["kv"]), q_pos0=d["q_pos0"], score_scale=d["score_scale"],
             sm_scale=d["sm_scale"])
    if q_rows is not None:
        h["q_rows"] = _u16(d["q"][torch.as_tensor(np.asarray(q_rows), device=d["q"].device)])
    return h


def check_prefill_sampled(dsa, d, h, out, lse, idx, rows, k, what, scores=True):
    """dsa_prefill's outputs on the given rows against the oracle, all rows per oracle call:
    the GPU's indexer score row of each (dsa_index_scores of that one query), its selection by
    the near-tie rule, its output and lse against the oracle's sparse MLA on the GPU's own
    indices.  Returns the statistics (also the number of near-tie swaps)."""
    rows = np.asarray(rows, np.int64)
    dev_rows = torch.as_tensor(rows, device=out.device)
    ora = oracle_rows(h, rows, k)
    gidx = _np(idx[dev_rows])
    swaps = check_indices_near_ties(gidx, ora["idx"], ora["scores"], ora["bound"], ora["n_vis"],
                                    k, what)
    q_rows = h["q_rows"] if "q_rows" in h else _u16(d["q"][dev_rows])
    oo, ol = oracle.sparse_mla(q_rows, h["kv"], gidx, h["sm_scale"])
    dout, rel, dl = check_mla(bf16_to_f64(out[dev_rows]), _np(lse[dev_rows]), oo, ol, what)
    stats = dict(rows_checked=int(len(rows)), near_tie_swaps=int(swaps), max_dout=dout,
                 max_rel_l2=rel, max_dlse=dl)
    if scores:
        worst = 0.0
        for i, t in enumerate(rows):
            t = int(t)
            g = dsa.dsa_index_scores(d["q8"][t:t + 1], d["qs"][t:t + 1], d["w"][t:t + 1],
                                     d["k8"], d["ks"], d["q_pos0"] + t, d["score_scale"])
            worst = max(worst, check_scores(_np(g), ora["scores"][i:i + 1],
                                            ora["bound"][i:i + 1], "%s scores row %d" % (what, t)))
        stats["max_dscore"] = worst
    return stats


def check_prefill_rows(d, out, lse, gidx, rows, k, what):
    ora = oracle_prefill_rows(d, rows, k)
    kv = _u16(d["kv"])
    swaps = 0
    for r in ora:
        t = r["t"]
        swaps += check_indices_near_ties(gidx[t:t + 1], r["idx"][None], r["scores"][None],
                                         r["bound"][None], [r["n"]], k, "%s row %d" % (what, t))
        oo, ol = oracle.sparse_mla(_u16(d["q"][t:t + 1]), kv, gidx[t:t + 1], d["sm_scale"])
        check_mla(bf16_to_f64(out[t:t + 1]), _np(lse[t:t + 1]), oo, ol, "%s row %d" % (what, t))
    return swaps


# ---------------------------------------------------------------- indexer warm-up (KL)
# Teacher logits are exact bf16 products summed in fp32; lse to 1e-4, P to 2e-3 relative.
# The gradient contractions round e = G * (key scale | w qs) * [x > 0] to bf16 (relative
# 2^-9) and accumulate in fp32, and G = Q - P itself carries fp32 error relative to Q + P:
# hence |delta| <= 2^-8 bnd + amb, with bnd the oracle's sum of |terms| with Q + P >= |G| in
# place of G, and amb the terms whose ReLU decision a rounded x may flip.  dw is accumulated
# in fp32 from unrounded e: 1e-3 of its bound.  kl: an error dI in the scores moves kl by
# sum_s G dI (|G| sums to <= 2) and P's relative error by that fraction of kl_bnd.
WU_LSE_ATOL = 1e-4
WU_P_RTOL = 2e-3
WU_GRAD_REL = 2.0 ** -8
WU_DW_REL = 1e-3
WU_KL_ATOL, WU_KL_REL = 5e-4, 1e-3
WU_LSEI_ATOL = 1e-3


def check_warmup_rows(g: dict, o: dict, rows_g, what=""):
    """GPU warm-up outputs (numpy, rows rows_g of them) against the oracle's rows.  Returns
    the worst error / tolerance ratio of each output."""
    worst = {}
    r = np.asarray(rows_g)
    dl = np.abs(g["lse_teacher"][r] - o["lse_t"])
    assert dl.max(initial=0) <= WU_LSE_ATOL, "%s: teacher lse off by %.3g" % (what, dl.max())
    worst["lse_teacher"] = dl.max(initial=0) / WU_LSE_ATOL
    di = np.abs(g["lse_index"][r] - o["lse_i"])
    assert di.max(initial=0) <= WU_LSEI_ATOL, "%s: index lse off by %.3g" % (what, di.max())
    worst["lse_index"] = di.max(initial=0) / WU_LSEI_ATOL
    dk_ = np.abs(g["kl"][r] - o["kl"])
    tol = WU_KL_ATOL + WU_KL_REL * o["kl_bnd"]
    assert (dk_ <= tol).all(), "%s: kl off by %.3g (tol %.3g)" % (what, dk_.max(), tol[np.argmax(dk_)])
    worst["kl"] = (dk_ / tol).max(initial=0)
    floor = 1e-7 * max(1.0, o["dq_bnd"].max(initial=0))
    d = np.abs(g["dq"][r] - o["dq"])
    tol = WU_GRAD_REL * o["dq_bnd"] + o["dq_amb"] + floor
    bad = d > tol
    assert not bad.any(), "%s: %d dq entries out of tolerance, worst %.3g (tol %.3g)" % (
        what, bad.sum(), d[bad].max(), tol[bad][np.argmax(d[bad])])
    worst["dq"] = (d / tol).max(initial=0)
    d = np.abs(g["dw"][r] - o["dw"])
    tol = WU_DW_REL * o["dw_bnd"] + 1e-9
    bad = d > tol
    assert not bad.any(), "%s: %d dw entries out of tolerance, worst %.3g" % (what, bad.sum(), d[bad].max())
    worst["dw"] = (d / tol).max(initial=0)
    return worst


def check_warmup_dk(g_dk: np.ndarray, o: dict, what=""):
    floor = 1e-7 * max(1.0, o["dk_bnd"].max(initial=0))
    d = np.abs(g_dk - o["dk"])
    tol = WU_GRAD_REL * o["dk_bnd"] + o["dk_amb"] + floor
    bad = d > tol
    assert not bad.any(), "%s: %d dk entries out of tolerance, worst %.3g (tol %.3g)" % (
        what, bad.sum(), d[bad].max(), tol[bad][np.argmax(d[bad])])
    return (d / tol).max(initial=0)


def _worker_count() -> int:
    """Host threads for per-sequence oracle calls: the CPUs this process may use, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _single_threaded_oracle():
    """Make the calling thread's OpenMP regions (inside the oracle library) use one thread, so
    that many Python threads can each run one sequence's oracle call side by side."""
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(1)
    except OSError:
        pass


def check_decode(dsa, inp, seqs, what):
    """One dsa_decode call over a packed batch; sequences `seqs` against the oracle: indices
    by the near-tie rule, output and lse against the oracle's sparse MLA on the GPU's
    indices.  Sequences are checked on a pool of host threads (one oracle call per sequence
    each).  Returns the statistics."""
    from concurrent.futures import ThreadPoolExecutor
    d = inp if inp["q"].is_cuda else to_device(inp)
    B, k = inp["B"], inp["k"]
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_decode(d["seq_start"], inp["max_len"], d["q8"], d["qs"], d["w"],
                                 d["k8"], d["ks"], d["q"], d["kv"], k, inp["score_scale"],
                                 inp["sm_scale"], idx_out=idx)
    torch.cuda.synchronize()
    st = _np(d["seq_start"])
    gidx = _np(idx)
    q8, qs, w, k8, ks = (_np(d[key]) for key in ("q8", "qs", "w", "k8", "ks"))
    q, kv = _u16(d["q"]), _u16(d["kv"])
    gout, glse = bf16_to_f64(out), _np(lse)

    def one(b):
        _single_threaded_oracle()
        a, e = int(st[b]), int(st[b + 1])
        Lb = e - a
        sc, bd = oracle.index_scores(q8[b:b + 1], qs[b:b + 1], w[b:b + 1], k8[a:e], ks[a:e],
                                     Lb - 1, inp["score_scale"], with_bound=True)
        oidx = oracle.topk(sc, [Lb], k)
        sw = check_indices_near_ties(gidx[b:b + 1], oidx, sc, bd, [Lb], k,
                                     "%s seq %d" % (what, b))
        oo, ol = oracle.sparse_mla(q[b:b + 1], kv[a:e], gidx[b:b + 1], inp["sm_scale"])
        errs = check_mla(gout[b:b + 1], glse[b:b + 1], oo, ol, "%s seq %d" % (what, b))
        return sw, errs

    with ThreadPoolExecutor(max_workers=_worker_count()) as ex:
        res = list(ex.map(one, list(seqs)))
    return dict(seqs_checked=len(res), near_tie_swaps=int(sum(r[0] for r in res)),
                max_dout=max((r[1][0] for r in res), default=0.0),
                max_rel_l2=max((r[1][1] for r in res), default=0.0),
                max_dlse=max((r[1][2] for r in res), default=0.0))
