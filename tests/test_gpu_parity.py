"""HIP path vs the CPU oracle, element by element, through the C ABI (needs an MI355X).

Small cases compare every row; the long workloads (32K and 128K prefill, 64-sequence decode)
run in the benchmark's launch configuration and compare sampled rows the oracle computes one
by one.  Tolerances: tests/parity.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (check_decode, check_indices_near_ties, check_mla, check_prefill_sampled,
                    check_scores, check_topk_exact, bf16_to_f64, host_prefill, report, to_device)
from synth import WORKLOADS, DecodeCfg, PrefillCfg, host_arrays, make_decode, make_prefill

pytestmark = pytest.mark.gpu


def _cfg(L, k, H_I, H, seed, q_pos0=0, T=None, planted=0.0):
    return PrefillCfg("case", L=L, k=k, H_I=H_I, H=H, w_std=H_I ** -0.5, seed=seed,
                      q_pos0=q_pos0, T=T, planted_frac=planted)


def _np(t):
    return t.detach().cpu().numpy()


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- indexer

@pytest.mark.parametrize("H_I,L,q_pos0,T", [
    (4, 1024, 0, None), (1, 300, 0, None), (2, 257, 5, 200), (8, 300, 0, None),
    (16, 200, 0, None), (32, 257, 10, 100), (64, 513, 0, None), (128, 130, 0, None),
    (64, 1, 0, None), (4, 17, 16, 1)])
def test_indexer_parity(dsa, H_I, L, q_pos0, T):
    cfg = _cfg(L, 16, H_I, 16, seed=100 + H_I + L, q_pos0=q_pos0, T=T)
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    g = dsa.dsa_index_scores(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], q_pos0, cfg.score_scale)
    torch.cuda.synchronize()
    o, bound = oracle.index_scores(h["q8"], h["qs"], h["w"], h["k8"], h["ks"], q_pos0,
                                   cfg.score_scale, with_bound=True)
    check_scores(_np(g), o, bound, "indexer H_I=%d L=%d" % (H_I, L))


def test_indexer_leading_dimension_leaves_padding_untouched(dsa):
    cfg = _cfg(200, 16, 64, 16, seed=7)
    inp = to_device(make_prefill(cfg))
    buf = torch.full((200, 256), 12345.0, device="cuda")
    dsa.dsa_index_scores(inp["q8"], inp["qs"], inp["w"], inp["k8"], inp["ks"], 0,
                         cfg.score_scale, scores=buf)
    torch.cuda.synchronize()
    assert torch.all(buf[:, 200:] == 12345.0)
    ref = dsa.dsa_index_scores(inp["q8"], inp["qs"], inp["w"], inp["k8"], inp["ks"], 0,
                               cfg.score_scale)
    assert torch.equal(buf[:, :200], ref)


def test_indexer_dense_heads_sampled_rows(dsa):
    """64 heads at L=2048: the shape of the dense-fallback workload."""
    cfg = WORKLOADS["prefill-L2048-k2048-dense"]
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    g = _np(dsa.dsa_index_scores(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], 0, cfg.score_scale))
    rows = np.array([0, 1, 15, 16, 17, 500, 1023, 1024, 2046, 2047])
    o, bound = oracle.index_scores(h["q8"], h["qs"], h["w"], h["k8"], h["ks"], 0,
                                   cfg.score_scale, rows=rows, with_bound=True)
    check_scores(g[rows], o, bound, "indexer L=2048 H_I=64")


@pytest.mark.parametrize("H_I", [4, 64])
@pytest.mark.parametrize("q_pos0,T", [(16000, 1000), (32500, 7500)])
def test_indexer_many_key_ranges(dsa, H_I, q_pos0, T):
    """Rows of 16,001 keys and more against a 40,000-key cache, split by the kernel over
    32,768-key ranges (grid.y) with 128-key tiles and causal early exit: full score rows
    compared element by element on rows whose visible ends straddle tile and range
    boundaries (16,384 and 32,768), with q_pos0 > 0."""
    L = 40000
    cfg = _cfg(L, 16, H_I, 16, seed=300 + H_I + q_pos0, q_pos0=q_pos0, T=T)
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    g = dsa.dsa_index_scores(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], q_pos0, cfg.score_scale)
    torch.cuda.synchronize()
    edges = [16255, 16256, 16383, 16384, 16385, 16511, 16512, 32639, 32640, 32767, 32768,
             32769, 32895, 32896, 39998, 39999]
    pos = [p for p in edges if q_pos0 <= p < q_pos0 + T] + [q_pos0, q_pos0 + 1, q_pos0 + T - 1]
    rng = np.random.default_rng(H_I + q_pos0)
    rows = np.unique(np.array(pos + rng.integers(q_pos0, q_pos0 + T, 24).tolist()) - q_pos0)
    o, bound = oracle.index_scores(h["q8"], h["qs"], h["w"], h["k8"], h["ks"], q_pos0,
                                   cfg.score_scale, rows=rows, with_bound=True)
    err = check_scores(_np(g[torch.from_numpy(rows).cuda()]), o, bound,
                       "indexer L=%d q_pos0=%d H_I=%d" % (L, q_pos0, H_I))
    report("indexer-L40000-q_pos0-%d-H_I%d" % (q_pos0, H_I), rows_checked=int(len(rows)),
           max_dscore=err)


# ----------------------------------------------------------------------------- top-k

def test_topk_exact_on_gpu_scores(dsa):
    cfg = WORKLOADS["prefill-L1024-k256"]
    d = to_device(make_prefill(cfg))
    s = dsa.dsa_index_scores(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], 0, cfg.score_scale)
    idx = dsa.dsa_topk(s, cfg.L, 0, cfg.k)
    torch.cuda.synchronize()
    check_topk_exact(_np(idx), _np(s), np.arange(cfg.L) + 1, cfg.k, "top-k L=1024")


@pytest.mark.parametrize("k", [1, 7, 64, 299, 300, 301, 8192])
def test_topk_ties_signed_zeros_and_k_edges(dsa, k):
    rng = np.random.default_rng(k)
    T, L, q_pos0 = 64, 300, 236
    vals = np.array([0.0, -0.0, 1.0, 1.0, 2.0, -1.0, 0.5], np.float32)
    s = rng.choice(vals, size=(T, L)).astype(np.float32)
    s[1] = 0.0
    s[2] = -0.0
    s[3] = rng.standard_normal(L).astype(np.float32)
    s[4, ::2] = -np.inf                                  # masked-looking values are still ranked
    g = torch.from_numpy(s).cuda()
    idx = dsa.dsa_topk(g, L, q_pos0, k)
    torch.cuda.synchronize()
    check_topk_exact(_np(idx), s, np.minimum(L, q_pos0 + np.arange(T) + 1), k, "ties k=%d" % k)


def test_topk_long_rows(dsa):
    rng = np.random.default_rng(5)
    T, L, k = 6, 40000, 2048
    s = rng.standard_normal((T, L)).astype(np.float32)
    s[1] = np.round(s[1] * 8) / 8                      # coarse values: ties at the threshold
    s[2] = 0.0
    g = torch.from_numpy(s).cuda()
    idx = dsa.dsa_topk(g, L, L - T, k)
    torch.cuda.synchronize()
    check_topk_exact(_np(idx), s, L - T + np.arange(T) + 1, k, "long rows")


def test_topk_threshold_estimate_misses_fall_back_exactly(dsa):
    """Rows whose sampled blocks are unrepresentative: the estimated threshold keeps too
    few (or too many) candidates and the row must take the exact path."""
    T, L, k = 4, 40000, 2048
    rng = np.random.default_rng(11)
    s = np.empty((T, L), np.float32)
    pos = np.arange(L)
    s[0] = -pos * 1e-3                                    # decreasing ...
    for blk in range(64):                                 # ... with the sampled blocks high
        start = blk * (L - 64) // 63
        s[0, start:start + 64] = 100.0 + rng.random(64)
    s[1] = np.where(pos % 2 == 0, 1.0, 0.0)               # massive ties at the threshold
    s[2] = rng.standard_normal(L)
    s[2, rng.choice(L, 3000, replace=False)] = 50.0       # many equal top values
    s[3] = -s[0]
    g = torch.from_numpy(s).cuda()
    idx = dsa.dsa_topk(g, L, L - T, k)
    torch.cuda.synchronize()
    check_topk_exact(_np(idx), s, L - T + np.arange(T) + 1, k, "estimate misses")


# -------------------------------------------------------------------------- sparse MLA

def _random_idx(T, L, k, q_pos0, rng, holes=True):
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(L, q_pos0 + t + 1)
        m = min(n, k)
        sel = rng.choice(n, size=m, replace=False).astype(np.int32)
        if holes and m < k:
            slots = np.sort(rng.choice(k, size=m, replace=False))
            idx[t, slots] = sel
        else:
            idx[t, :m] = sel
    return idx


@pytest.mark.parametrize("H,L,k", [(8, 1024, 256), (16, 300, 64), (128, 600, 100),
                                   (40, 200, 33), (128, 3000, 2048)])
def test_sparse_mla_parity(dsa, H, L, k):
    cfg = _cfg(L, k, 4, H, seed=H * 7 + k, T=min(L, 160), q_pos0=L - min(L, 160))
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    idx = _random_idx(cfg.rows, L, k, cfg.q_pos0, np.random.default_rng(H))
    out, lse = dsa.dsa_sparse_mla(d["q"], d["kv"], torch.from_numpy(idx).cuda(), cfg.sm_scale)
    torch.cuda.synchronize()
    oo, ol = oracle.sparse_mla(h["q"], h["kv"], idx, cfg.sm_scale)
    check_mla(bf16_to_f64(out), _np(lse), oo, ol, "mla H=%d L=%d k=%d" % (H, L, k))


@pytest.mark.parametrize("L,k", [(9000, 6000), (8300, 8192)])
def test_sparse_mla_long_index_lists(dsa, L, k):
    """Index lists longer than the kernel's 4096-key validity segment (two segments, padding
    holes in both): every row against the oracle."""
    cfg = _cfg(L, k, 4, 128, seed=k, T=4, q_pos0=L - 4)
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    idx = _random_idx(cfg.rows, L, k, cfg.q_pos0, np.random.default_rng(k))
    idx[:, ::7] = -1                                   # holes in every 32-key tile
    out, lse = dsa.dsa_sparse_mla(d["q"], d["kv"], torch.from_numpy(idx).cuda(), cfg.sm_scale)
    torch.cuda.synchronize()
    oo, ol = oracle.sparse_mla(h["q"], h["kv"], idx, cfg.sm_scale)
    check_mla(bf16_to_f64(out), _np(lse), oo, ol, "mla long L=%d k=%d" % (L, k))


def test_sparse_mla_rows_at_the_cache_limit(dsa):
    """The gather finds a row by its byte offset in the cache: a cache of 1,864,135 rows (the
    2 GiB the entry points accept), index lists drawn from its last rows and from across it,
    against the oracle on a compact copy of the selected rows (indices remapped)."""
    L, T, H, k = 1864135, 3, 16, 96
    g = torch.Generator(device="cuda").manual_seed(41)
    kv = (torch.randn((L, 576), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    q = (torch.randn((T, H, 576), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    rng = np.random.default_rng(41)
    idx = np.empty((T, k), np.int32)
    idx[0] = np.arange(L - k, L)                               # the last rows
    idx[1] = rng.choice(L, k, replace=False)                   # across the cache
    idx[2] = np.concatenate([np.arange(L - 32, L), rng.choice(L - 32, k - 32, replace=False)])
    sm_scale = 576 ** -0.5
    out, lse = dsa.dsa_sparse_mla(q, kv, torch.from_numpy(idx).cuda(), sm_scale)
    torch.cuda.synchronize()
    uniq, inv = np.unique(idx, return_inverse=True)
    kv_c = _u16(kv[torch.from_numpy(uniq).long().cuda()])
    idx_c = inv.reshape(idx.shape).astype(np.int32)
    oo, ol = oracle.sparse_mla(_u16(q), kv_c, idx_c, sm_scale)
    check_mla(bf16_to_f64(out), _np(lse), oo, ol, "mla rows at the cache limit")
    del kv
    torch.cuda.empty_cache()


def test_sparse_mla_late_dominant_logit_recomputes(dsa):
    """The kernel fixes each head's softmax reference from the first valid logits and
    recomputes the row with the exact maximum when a later logit exceeds that reference by
    more than 2^64 in the exp2 domain.  Here the first 32 selected keys have logits of order
    1 and a key late in the list has logit 96 for every head: results must still match the
    oracle (and be finite)."""
    L, k, T, H = 200, 100, 3, 128
    cfg = _cfg(L, k, 4, H, seed=11, T=T, q_pos0=L - T)
    inp = make_prefill(cfg)
    inp["q"] = torch.full_like(inp["q"], 2.0)          # q . kv[big] = 2 * 2 * 576 = 2304
    kv = inp["kv"].clone()
    kv[150] = 2.0
    inp["kv"] = kv
    h, d = host_arrays(inp), to_device(inp)
    rng = np.random.default_rng(5)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        sel = rng.choice(np.setdiff1d(np.arange(L - T + t + 1), [150]), size=k - 1, replace=False)
        idx[t, :k - 1] = sel
        idx[t, 60 + t] , idx[t, k - 1] = 150, idx[t, 60 + t]   # key 150 at position 60 + t
    out, lse = dsa.dsa_sparse_mla(d["q"], d["kv"], torch.from_numpy(idx).cuda(), cfg.sm_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    oo, ol = oracle.sparse_mla(h["q"], h["kv"], idx, cfg.sm_scale)
    check_mla(bf16_to_f64(out), _np(lse), oo, ol, "mla late dominant logit")


def test_sparse_mla_single_row_closed_form_and_empty_rows(dsa):
    """A row selecting only token 0 returns kv[0, :512] exactly (softmax weight 1); a row
    with no valid index (all -1 or out of range) returns zeros and lse = -inf."""
    cfg = _cfg(64, 8, 4, 32, seed=3)
    d = to_device(make_prefill(cfg))
    idx = torch.full((64, 8), -1, dtype=torch.int32)
    idx[0, 3] = 0
    idx[2, :] = 64                                     # out of range -> padding
    idx[3, 5] = 1000
    idx[5, :] = torch.arange(8)
    out, lse = dsa.dsa_sparse_mla(d["q"], d["kv"], idx.cuda(), cfg.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out[0], d["kv"][0, :512].unsqueeze(0).expand(32, 512))
    ref = (d["q"][0].double() @ d["kv"][0].double()) * cfg.sm_scale
    assert torch.allclose(lse[0].double(), ref, atol=1e-4, rtol=1e-5)
    for r in (1, 2, 3, 4):
        assert torch.all(out[r].float() == 0) and torch.all(torch.isneginf(lse[r]))


# ------------------------------------------------------------------- prefill, end to end

def test_prefill_small_every_row(dsa):
    cfg = WORKLOADS["prefill-L1024-k256"]
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    idx = torch.empty((cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_prefill(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                  cfg.k, 0, cfg.score_scale, cfg.sm_scale, idx_out=idx)
    torch.cuda.synchronize()
    ref = oracle.prefill(h, with_bound=True)
    gidx = _np(idx)
    swaps = check_indices_near_ties(gidx, ref["idx"], ref["scores"], ref["bound"], ref["n_vis"],
                                    cfg.k, "prefill L=1024")
    oo, ol = oracle.sparse_mla(h["q"], h["kv"], gidx, cfg.sm_scale)
    e = check_mla(bf16_to_f64(out), _np(lse), oo, ol, "prefill L=1024")
    report(cfg.name, rows_checked=cfg.L, near_tie_swaps=int(swaps), max_dout=e[0],
           max_rel_l2=e[1], max_dlse=e[2])


def test_prefill_dense_fallback_equals_dense_attention(dsa):
    """Every row sees <= k = 2048 tokens: the selection is everything and the output is
    exact causal attention (every row against the dense oracle)."""
    cfg = WORKLOADS["prefill-L2048-k2048-dense"]
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    idx = torch.empty((cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_prefill(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                  cfg.k, 0, cfg.score_scale, cfg.sm_scale, idx_out=idx)
    torch.cuda.synchronize()
    gidx = _np(idx)
    want = np.where(np.arange(cfg.k)[None, :] <= np.arange(cfg.L)[:, None],
                    np.arange(cfg.k)[None, :], -1)
    assert np.array_equal(gidx, want)
    do, dl = oracle.dense_mla(h["q"], h["kv"], 0, cfg.sm_scale)
    e = check_mla(bf16_to_f64(out), _np(lse), do, dl, "dense fallback")
    report(cfg.name, rows_checked=cfg.L, near_tie_swaps=0, max_dout=e[0], max_rel_l2=e[1],
           max_dlse=e[2])


def test_prefill_chunk_with_q_pos0_matches_full(dsa):
    cfg = _cfg(700, 96, 64, 32, seed=44)
    d = to_device(make_prefill(cfg))
    args = lambda sl: (d["q8"][sl], d["qs"][sl], d["w"][sl], d["k8"], d["ks"], d["q"][sl], d["kv"])
    full_idx = torch.empty((700, 96), dtype=torch.int32, device="cuda")
    fo, fl, _ = dsa.dsa_prefill(*args(slice(0, 700)), 96, 0, cfg.score_scale, cfg.sm_scale,
                                idx_out=full_idx)
    part_idx = torch.empty((450, 96), dtype=torch.int32, device="cuda")
    po, pl, _ = dsa.dsa_prefill(*args(slice(250, 700)), 96, 250, cfg.score_scale, cfg.sm_scale,
                                idx_out=part_idx)
    torch.cuda.synchronize()
    assert torch.equal(full_idx[250:], part_idx)
    assert torch.equal(fo[250:], po) and torch.equal(fl[250:], pl)


def test_prefill_bitwise_repeatable(dsa):
    cfg = _cfg(1500, 256, 64, 64, seed=9)
    d = to_device(make_prefill(cfg))
    outs = []
    for _ in range(2):
        idx = torch.empty((1500, 256), dtype=torch.int32, device="cuda")
        o, l, _ = dsa.dsa_prefill(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                  256, 0, cfg.score_scale, cfg.sm_scale, idx_out=idx)
        outs.append((o.clone(), l.clone(), idx.clone()))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def _sampled_rows(L, k, planted, n, seed):
    """At least n rows: the fixed edge rows, the target rows of up to 64 planted tokens, and
    the rest uniform from a fixed seed."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, k - 2, k - 1, k, k + 1, L - 2, L - 1]
    tgt = [int(t) for t in planted[:, 1][:64]] if len(planted) else []
    rows = np.unique(np.array(fixed + tgt))
    while len(rows) < n:
        rows = np.unique(np.concatenate([rows, rng.integers(0, L, n - len(rows))]))
    return rows


@pytest.mark.parametrize("name", ["prefill-L32768-k2048", "prefill-L131072-k2048"])
def test_prefill_long_context_sampled_rows(dsa, name):
    """The long workloads in the benchmark's launch configuration: on 256 sampled rows the
    GPU's full indexer score row, its selection (near-tie rule) and its output; every planted
    token against the row it was aimed at (recall, misses checked against the oracle); and the
    standalone top-k exactly against the oracle on full-length rows of GPU scores."""
    cfg = WORKLOADS[name]
    d = make_prefill(cfg, device="cuda")
    idx = torch.empty((cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_prefill(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                  cfg.k, 0, cfg.score_scale, cfg.sm_scale, idx_out=idx)
    torch.cuda.synchronize()
    planted = _np(d["planted"])
    rows = _sampled_rows(cfg.L, cfg.k, planted, 256, cfg.seed)
    h = host_prefill(d, q_rows=rows)
    stats = check_prefill_sampled(dsa, d, h, out, lse, idx, rows, cfg.k, name)

    # planted tokens: found by the rows they were aimed at, or else not selected by the
    # oracle either / a near-tie there
    tgt = torch.from_numpy(planted[:, 1].astype(np.int64)).cuda()
    sel = _np(idx[tgt])
    hit = np.array([s in set(r.tolist()) for s, r in zip(planted[:, 0], sel)])
    miss = np.nonzero(~hit)[0]
    if len(miss):
        from parity import oracle_rows
        o = oracle_rows(h, planted[miss, 1], cfg.k)
        for j, m in enumerate(miss):
            s = int(planted[m, 0])
            if s in set(o["idx"][j].tolist()):
                n = int(o["n_vis"][j])
                row = o["scores"][j, :n]
                tau = np.sort(row)[::-1][cfg.k - 1]
                tol = 1e-3 * abs(tau) + 2.0 ** -16 * o["bound"][j, :n].max()
                assert abs(row[s] - tau) <= tol, "planted key %d missed by row %d" % (
                    s, planted[m, 1])
    stats["planted"] = int(len(planted))
    stats["planted_recall"] = float(hit.mean()) if len(hit) else None

    # standalone top-k on the GPU's own scores of full-length rows (the last rows see every
    # key; rows in the middle see about half of them): exact set equality
    T = 4
    exact = 0
    for p0 in (cfg.L - T, cfg.L // 2):
        sc = dsa.dsa_index_scores(d["q8"][p0:p0 + T], d["qs"][p0:p0 + T], d["w"][p0:p0 + T],
                                  d["k8"], d["ks"], p0, cfg.score_scale)
        tk = dsa.dsa_topk(sc, cfg.L, p0, cfg.k)
        torch.cuda.synchronize()
        check_topk_exact(_np(tk), _np(sc), p0 + np.arange(T) + 1, cfg.k,
                         "%s top-k rows %d.." % (name, p0))
        exact += T
    stats["topk_exact_full_rows"] = exact
    report(name, **stats)
    del h


# ---------------------------------------------------------------------------- decode

@pytest.mark.parametrize("B,lo,hi,k,H_I,H", [(8, 1, 9000, 2048, 64, 128), (5, 3, 700, 64, 4, 16),
                                             (3, 1, 40, 8, 128, 8)])
def test_decode_every_sequence(dsa, B, lo, hi, k, H_I, H):
    cfg = DecodeCfg("case", B=B, len_lo=lo, len_hi=hi, k=k, H_I=H_I, H=H, w_std=H_I ** -0.5,
                    seed=B * 31 + k)
    inp = make_decode(cfg)
    check_decode(dsa, inp, range(B), "decode B=%d k=%d" % (B, k))


def test_decode_64_sequences_to_128k_every_sequence(dsa):
    cfg = WORKLOADS["decode-B64-L4096-131072-k2048"]
    inp = make_decode(cfg, device="cuda")
    stats = check_decode(dsa, inp, range(cfg.B), "decode B=64")
    report(cfg.name, **stats)


def test_decode_sequence_longer_than_max_len_selects_nothing(dsa):
    """A sequence longer than the max_len the caller passes is outside the contract: it gets
    no selection (indices -1, output 0, lse -inf) instead of reading unscored positions, and
    the other sequences are unaffected."""
    cfg = DecodeCfg("case", B=4, len_lo=300, len_hi=3000, k=256, H_I=64, H=32, w_std=1 / 8,
                    seed=77)
    inp = make_decode(cfg)
    d = to_device(inp)
    lens = _np(inp["lens"])
    long_b = int(np.argmax(lens))
    short_max = int(np.sort(lens)[-2])                  # every other sequence still fits
    assert lens[long_b] > short_max
    args = lambda ml: (d["seq_start"], ml, d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"],
                       d["kv"], cfg.k, cfg.score_scale, cfg.sm_scale)
    idx_ok = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device="cuda")
    out_ok, lse_ok, _ = dsa.dsa_decode(*args(inp["max_len"]), idx_out=idx_ok)
    idx = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_decode(*args(short_max), idx_out=idx)
    torch.cuda.synchronize()
    assert torch.all(idx[long_b] == -1)
    assert torch.all(out[long_b].float() == 0) and torch.all(torch.isneginf(lse[long_b]))
    others = [b for b in range(cfg.B) if b != long_b]
    assert torch.equal(idx[others], idx_ok[others])
    assert torch.equal(out[others], out_ok[others]) and torch.equal(lse[others], lse_ok[others])


def _decode_integer_scores(vals_per_seq, k, H=8, seed=0):
    """Decode inputs whose indexer scores are exact small integers in any summation order:
    H_I = 1, a one-hot fp8 query (1.0 in dimension 0), key dimension 0 = the integer value
    (0..7, exact in e4m3), all other key dimensions 0, unit scales and weights."""
    g = torch.Generator().manual_seed(seed)
    lens = np.array([len(v) for v in vals_per_seq], np.int64)
    B, N = len(lens), int(lens.sum())
    st = np.zeros(B + 1, np.int64)
    st[1:] = np.cumsum(lens)
    code = torch.arange(8, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    vals = np.concatenate(vals_per_seq).astype(np.int64)
    k8 = torch.zeros((N, 128), dtype=torch.uint8)
    k8[:, 0] = code[torch.from_numpy(vals)]
    q8 = torch.zeros((B, 1, 128), dtype=torch.uint8)
    q8[:, :, 0] = code[1]
    inp = dict(B=B, N=N, H_I=1, H=H, k=k, max_len=int(lens.max()), lens=torch.from_numpy(lens),
               seq_start=torch.from_numpy(st), score_scale=1.0, sm_scale=0.05, q8=q8,
               qs=torch.ones((B, 1)), w=torch.ones((B, 1)), k8=k8, ks=torch.ones(N),
               q=torch.randn((B, H, 576), generator=g).to(torch.bfloat16),
               kv=torch.randn((N, 576), generator=g).to(torch.bfloat16))
    return inp, st, vals


def test_decode_topk_exact_on_integer_scores(dsa):
    """Decode rows that the top-k splits over 16K-key segments, with exact integer scores so
    that the selection (ties to the lower position) is compared exactly: ties at the
    threshold spread over several segments (the segments' candidates merged), a row of equal
    scores (segment candidate counts overflow: the exact path), a row staged whole, a row
    shorter than k, and rows whose threshold falls either way."""
    rng = np.random.default_rng(21)
    k = 2048
    r0 = rng.integers(0, 3, 40000)                      # 1000 sevens, 4000 sixes, rest 0..2
    p = rng.permutation(40000)
    r0[p[:1000]] = 7
    r0[p[1000:5000]] = 6
    r0[16383:16386] = 7                                 # around the first segment boundary
    r1 = np.zeros(20000, np.int64)                      # every score equal
    r2 = rng.integers(0, 8, 3000)                       # staged whole
    r3 = rng.integers(0, 8, 1500)                       # fewer keys than k
    r4 = rng.integers(0, 8, 33000)                      # about 4100 sevens
    r5 = (7 - np.arange(16385) * 8 // 16385).astype(np.int64)   # a ramp into segment 2
    inp, st, vals = _decode_integer_scores([r0, r1, r2, r3, r4, r5], k)
    d = to_device(inp)
    idx = torch.empty((inp["B"], k), dtype=torch.int32, device="cuda")
    dsa.dsa_decode(d["seq_start"], inp["max_len"], d["q8"], d["qs"], d["w"], d["k8"], d["ks"],
                   d["q"], d["kv"], k, 1.0, 0.05, idx_out=idx)
    torch.cuda.synchronize()
    gidx = _np(idx)
    for b in range(inp["B"]):
        sc = vals[st[b]:st[b + 1]].astype(np.float64)[None, :]
        want = oracle.topk(sc, [len(sc[0])], k)
        assert np.array_equal(gidx[b], want[0]), "decode top-k row %d (n=%d) differs" % (
            b, len(sc[0]))
