"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a library routine, a closed form, a hand-computed
example, brute force, or an invariant, so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import PrefillCfg, host_arrays, make_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- codecs

def test_e4m3fn_decoder_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_values(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2                      # 0x7F and 0xFF
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))   # -0 is 0x80


def test_bf16_decoder_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint16)
    mine = oracle.bf16_values(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


# ---------------------------------------------------------------------------- indexer

def _e4m3_deq(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)


def _small_prefill(L=48, H_I=1, H=2, k=8, seed=5, q_pos0=0, T=None):
    cfg = PrefillCfg("t", L=L, k=k, H_I=H_I, H=H, w_std=1.0, seed=seed, q_pos0=q_pos0, T=T)
    return host_arrays(make_prefill(cfg))


def test_indexer_single_head_is_relu_of_matmul():
    """H_I = 1, unit weights/scales: scores are ReLU(deq(q) @ deq(k)^T) under the causal
    mask.  fp64 matmul is exact here (products of e4m3 values span < 53 bits)."""
    a = _small_prefill(L=40, H_I=1, q_pos0=3, T=30)
    T, L = a["T"], a["L"]
    ones_t = np.ones((T, 1), np.float32)
    s = oracle.index_scores(a["q8"], ones_t, ones_t, a["k8"], np.ones(L, np.float32),
                            a["q_pos0"], 1.0)
    D = _e4m3_deq(a["q8"][:, 0, :]) @ _e4m3_deq(a["k8"]).T
    ref = torch.clamp(D, min=0).numpy()
    mask = np.arange(L)[None, :] > (a["q_pos0"] + np.arange(T))[:, None]
    ref[mask] = -np.inf
    assert np.array_equal(s, ref)


def test_indexer_single_head_scales_multiply():
    a = _small_prefill(L=33, H_I=1)
    c = 0.0883883
    s = oracle.index_scores(a["q8"], a["qs"], a["w"], a["k8"], a["ks"], 0, c)
    D = (_e4m3_deq(a["q8"][:, 0, :]) @ _e4m3_deq(a["k8"]).T).numpy()
    wp = a["w"][:, 0].astype(np.float64) * a["qs"][:, 0].astype(np.float64) * c
    ref = np.maximum(D, 0) * wp[:, None] * a["ks"].astype(np.float64)[None, :]
    vis = np.tril(np.ones_like(ref, dtype=bool))
    assert np.allclose(s[vis], ref[vis], rtol=1e-14, atol=0)
    assert np.all(np.isneginf(s[~vis]))


def test_indexer_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "indexer_hand.json")))
    enc = {float(v): c for v, c in g["e4m3fn_codes"].items()}
    enc[0.0] = 0
    T, H_I, L = g["T"], g["H_I"], g["L"]
    q8 = np.zeros((T, H_I, 128), np.uint8)
    k8 = np.zeros((L, 128), np.uint8)
    for t in range(T):
        for h in range(H_I):
            for d, v in enumerate(g["q_values"][t][h]):
                q8[t, h, d] = enc[v]
    for s in range(L):
        for d, v in enumerate(g["k_values"][s]):
            k8[s, d] = enc[v]
    got, bound = oracle.index_scores(q8, np.array(g["qs"], np.float32), np.array(g["w"], np.float32),
                                     k8, np.array(g["ks"], np.float32), g["q_pos0"], g["c"],
                                     with_bound=True)
    exp = np.array([[float(x) for x in row] for row in g["expected_scores"]])
    assert np.array_equal(got, exp)
    vis = np.isfinite(exp)
    assert np.all(bound[vis] >= np.abs(got[vis]))
    n_vis = g["q_pos0"] + np.arange(T) + 1
    assert oracle.topk(got, n_vis, 1).tolist() == g["expected_top1"]
    assert oracle.topk(got, n_vis, 2).tolist() == g["expected_top2"]


def test_indexer_power_of_two_scaling_is_exact():
    a = _small_prefill(L=40, H_I=4, seed=9)
    c = 0.125
    base = oracle.index_scores(a["q8"], a["qs"], a["w"], a["k8"], a["ks"], 0, c)
    s2 = oracle.index_scores(a["q8"], a["qs"], a["w"] * 2, a["k8"], a["ks"] * 4, 0, c / 8)
    assert np.array_equal(base, s2)          # 2 * 4 / 8 = 1, all exact in binary fp


def test_indexer_joint_head_permutation_invariance():
    a = _small_prefill(L=40, H_I=8, seed=11)
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    c = 0.1
    base = oracle.index_scores(a["q8"], a["qs"], a["w"], a["k8"], a["ks"], 0, c)
    p = oracle.index_scores(a["q8"][:, perm], a["qs"][:, perm], a["w"][:, perm], a["k8"],
                            a["ks"], 0, c)
    vis = np.isfinite(base)
    assert np.allclose(p[vis], base[vis], rtol=1e-13, atol=1e-13)
    # and a single-head split: score(heads) == sum over one-head calls
    acc = np.zeros_like(base)
    for h in range(8):
        acc += np.where(vis, oracle.index_scores(a["q8"][:, h:h + 1], a["qs"][:, h:h + 1],
                                                 a["w"][:, h:h + 1], a["k8"], a["ks"], 0, c), 0)
    assert np.allclose(acc[vis], base[vis], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("H_I,L,q_pos0,T,seed", [(4, 70, 0, None, 12), (64, 40, 9, 25, 13)])
def test_indexer_bound_many_heads_is_weighted_abs_einsum(H_I, L, q_pos0, T, seed):
    """The conditioning bound A[t,s] = ks[s] sum_h |w qs c| sum_d |q k| with several heads,
    written as a torch float64 abs-einsum over the dequantised codes (torch's fp8 cast, not the
    oracle's decoder).  Dropping the absolute value of a signed weight, a transposed head index
    or a missing key scale changes A; masked entries carry no bound."""
    a = _small_prefill(L=L, H_I=H_I, seed=seed, q_pos0=q_pos0, T=T)
    c = 0.0883883
    _, bound = oracle.index_scores(a["q8"], a["qs"], a["w"], a["k8"], a["ks"], q_pos0, c,
                                   with_bound=True)
    absdot = torch.einsum("thd,sd->ths", torch.abs(_e4m3_deq(a["q8"])),
                          torch.abs(_e4m3_deq(a["k8"]))).numpy()
    wp = np.abs(a["w"].astype(np.float64) * a["qs"].astype(np.float64) * c)       # [T, H_I]
    ref = np.einsum("th,ths->ts", wp, absdot) * a["ks"].astype(np.float64)[None, :]
    vis = np.arange(L)[None, :] <= (q_pos0 + np.arange(a["T"]))[:, None]
    assert np.allclose(bound[vis], ref[vis], rtol=1e-13, atol=0)
    assert np.all(bound[~vis] == 0.0)
    # the signed weights matter: with |w| the bound is unchanged, with w it is not
    assert (a["w"] < 0).any()


def test_indexer_bound_covers_fp32_evaluation_error():
    """The score tolerance floor 2^-16 A covers an fp32 evaluation of the same sum in another
    order (per-head fp32 dots, fp32 weighted head sum), at 64 heads where signed heads cancel."""
    a = _small_prefill(L=300, H_I=64, seed=14)
    c = 128 ** -0.5
    exact, bound = oracle.index_scores(a["q8"], a["qs"], a["w"], a["k8"], a["ks"], 0, c,
                                       with_bound=True)
    q = _e4m3_deq(a["q8"]).float()
    k = _e4m3_deq(a["k8"]).float()
    D = torch.einsum("thd,sd->ths", q, k)                                   # fp32
    wp = (torch.from_numpy(a["w"]) * torch.from_numpy(a["qs"]) * c).float()
    s32 = (torch.relu(D) * wp[:, :, None]).sum(1) * torch.from_numpy(a["ks"])[None, :]
    vis = np.isfinite(exact)
    err = np.abs(s32.double().numpy()[vis] - exact[vis])
    assert np.all(err <= 1e-3 * np.abs(exact[vis]) + 2.0 ** -16 * bound[vis])
    assert err.max() > 0                         # the fp32 evaluation really does round


def test_indexer_bound_single_head_is_abs_matmul():
    a = _small_prefill(L=20, H_I=1, seed=4)
    c = 0.3
    _, bound = oracle.index_scores(a["q8"], a["qs"], a["w"], a["k8"], a["ks"], 0, c, with_bound=True)
    absdot = (torch.abs(_e4m3_deq(a["q8"][:, 0, :])) @ torch.abs(_e4m3_deq(a["k8"])).T).numpy()
    wp = np.abs(a["w"][:, 0].astype(np.float64) * a["qs"][:, 0].astype(np.float64) * c)
    ref = absdot * wp[:, None] * a["ks"].astype(np.float64)[None, :]
    vis = np.tril(np.ones_like(ref, dtype=bool))
    assert np.allclose(bound[vis], ref[vis], rtol=1e-14, atol=0)


# ------------------------------------------------------------------------------ top-k

def _brute_topk(row, k):
    """The unique k-subset whose every member beats every non-member under
    (score descending, position ascending), found by enumeration."""
    n = len(row)
    if n <= k:
        return list(range(n))
    key = lambda s: (-row[s], s)
    found = []
    for sub in itertools.combinations(range(n), k):
        worst_in = max(key(s) for s in sub)
        rest = set(range(n)) - set(sub)
        if all(key(s) > worst_in for s in rest):
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_with_ties_and_signed_zeros(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.5, 2.5, 0.0])
    row = rng.choice(vals, size=n) if seed % 2 == 0 else rng.standard_normal(n)
    for k in range(1, n + 2):
        want = _brute_topk(list(row), k)
        want = want + [-1] * (k - len(want))
        for m in ("sort", "select"):
            got = oracle.topk(row[None, :], [n], k, method=m)[0].tolist()
            assert got == want, (m, row, k)


def test_topk_matches_torch_stable_sort_and_both_selectors_agree():
    rng = np.random.default_rng(3)
    rows = 40
    L = 600
    s = rng.standard_normal((rows, L))
    s[::3] = np.round(s[::3] * 4) / 4          # heavy ties on some rows
    s[1, :] = 0.0
    s[1, ::2] = -0.0                           # -0 and +0 must tie
    n_vis = rng.integers(1, L + 1, rows)
    k = 64
    a = oracle.topk(s, n_vis, k, "sort")
    b = oracle.topk(s, n_vis, k, "select")
    assert np.array_equal(a, b)
    for r in range(rows):
        n = n_vis[r]
        if n <= k:
            assert a[r].tolist() == list(range(n)) + [-1] * (k - n)
            continue
        order = torch.sort(torch.from_numpy(-s[r, :n]), stable=True).indices[:k]
        assert a[r].tolist() == sorted(order.tolist())


def test_topk_invariants():
    rng = np.random.default_rng(7)
    L, k = 3000, 100
    s = rng.standard_normal((8, L))
    n_vis = np.array([1, 50, 100, 101, 2000, 2999, 3000, 700])
    idx = oracle.topk(s, n_vis, k)
    for r in range(8):
        n = n_vis[r]
        sel = idx[r][idx[r] >= 0]
        assert len(sel) == min(n, k)
        assert len(set(sel.tolist())) == len(sel)
        assert np.all(sel < n)
        assert np.argmax(s[r, :n]) in sel
        if n > k:
            rest = np.setdiff1d(np.arange(n), sel)
            assert s[r, sel].min() >= s[r, rest].max()


# -------------------------------------------------------------------------------- MLA

def _bf16(x):
    return torch.as_tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _deq16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def test_mla_first_row_closed_form():
    """Row at position 0 selects only token 0: out is kv[0, :512] exactly and
    lse = sm_scale * <q, kv[0]>."""
    a = _small_prefill(L=16, H=4, k=4, seed=2)
    idx = np.full((a["T"], 4), -1, np.int32)
    idx[0, 2] = 0
    out, lse = oracle.sparse_mla(a["q"], a["kv"], idx, 0.05, rows=[0])
    kv0 = _deq16(a["kv"][0]).numpy()
    assert np.array_equal(out[0], np.broadcast_to(kv0[:512], (4, 512)))
    qd = _deq16(a["q"][0]).numpy()
    assert np.allclose(lse[0], 0.05 * (qd @ kv0), rtol=1e-14)


def test_mla_zero_query_is_mean_of_selected_rows():
    a = _small_prefill(L=30, H=2, k=6, seed=3)
    q = np.zeros_like(a["q"])
    idx = np.array([[3, 17, -1, 0, 29, 8]], np.int32).repeat(a["T"], 0)
    out, lse = oracle.sparse_mla(q, a["kv"], idx, 0.1, rows=[5])
    sel = [3, 17, 0, 29, 8]
    mean = _deq16(a["kv"][sel]).numpy()[:, :512].mean(0)
    assert np.allclose(out[0], mean[None, :], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse[0], math.log(5), rtol=1e-14)


def _sdpa_ref(q_bits, kv_bits, q_pos0, sm_scale):
    q = _deq16(q_bits).permute(1, 0, 2).unsqueeze(0)          # [1, H, T, 576]
    kv = _deq16(kv_bits)
    T, L = q.shape[2], kv.shape[0]
    mask = torch.arange(L)[None, :] <= (q_pos0 + torch.arange(T))[:, None]
    K = kv.unsqueeze(0).unsqueeze(0).expand(1, q.shape[1], L, 576).contiguous()
    V = kv[:, :512].unsqueeze(0).unsqueeze(0).expand(1, q.shape[1], L, 512).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=sm_scale)
    logits = (q @ K.transpose(-1, -2)) * sm_scale
    lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
    return o[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def test_dense_mla_matches_torch_sdpa():
    a = _small_prefill(L=70, H=4, k=8, seed=8, q_pos0=20, T=50)
    out, lse = oracle.dense_mla(a["q"], a["kv"], a["q_pos0"], a["sm_scale"])
    ro, rl = _sdpa_ref(a["q"], a["kv"], a["q_pos0"], a["sm_scale"])
    assert np.allclose(out, ro, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_sparse_mla_with_all_visible_equals_dense_and_sdpa():
    a = _small_prefill(L=40, H=2, k=64, seed=12)
    T = a["T"]
    idx = np.full((T, 64), -1, np.int32)
    rng = np.random.default_rng(0)
    for t in range(T):
        perm = rng.permutation(t + 1)                 # order within a row must not matter
        slots = rng.choice(64, size=t + 1, replace=False)
        idx[t, slots] = perm
    so, sl = oracle.sparse_mla(a["q"], a["kv"], idx, a["sm_scale"])
    do, dl = oracle.dense_mla(a["q"], a["kv"], 0, a["sm_scale"])
    assert np.allclose(so, do, rtol=1e-12, atol=1e-13)
    assert np.allclose(sl, dl, rtol=1e-13, atol=1e-13)
    ro, rl = _sdpa_ref(a["q"], a["kv"], 0, a["sm_scale"])
    assert np.allclose(so, ro, rtol=1e-10, atol=1e-12)


def test_sparse_mla_subset_matches_masked_sdpa():
    """An arbitrary index set is attention with every other key masked out."""
    a = _small_prefill(L=50, H=3, k=10, seed=13)
    rng = np.random.default_rng(1)
    T = a["T"]
    idx = np.full((T, 10), -1, np.int32)
    mask = np.zeros((T, 50), bool)
    for t in range(T):
        m = min(10, t + 1)
        sel = rng.choice(t + 1, size=m, replace=False)
        idx[t, :m] = sel
        mask[t, sel] = True
    out, lse = oracle.sparse_mla(a["q"], a["kv"], idx, 0.07)
    q = _deq16(a["q"]).permute(1, 0, 2).unsqueeze(0)
    kv = _deq16(a["kv"])
    K = kv.expand(3, 50, 576).unsqueeze(0).contiguous()
    V = kv[:, :512].expand(3, 50, 512).unsqueeze(0).contiguous()
    ro = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=torch.from_numpy(mask), scale=0.07)
    assert np.allclose(out, ro[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------- composed paths

def test_prefill_short_context_equals_dense_attention():
    """Every row sees <= k tokens: DSA selects everything and equals full attention."""
    cfg = PrefillCfg("t", L=24, k=32, H_I=4, H=2, w_std=0.5, seed=21)
    a = host_arrays(make_prefill(cfg))
    res = oracle.prefill(a)
    for t in range(a["T"]):
        assert res["idx"][t].tolist() == list(range(t + 1)) + [-1] * (32 - t - 1)
    do, dl = oracle.dense_mla(a["q"], a["kv"], 0, a["sm_scale"])
    assert np.allclose(res["out"], do, rtol=1e-12, atol=1e-13)
    assert np.allclose(res["lse"], dl, rtol=1e-13, atol=1e-13)


def test_decode_matches_prefill_last_row_and_dense_when_short():
    from synth import DecodeCfg, make_decode
    cfg = DecodeCfg("t", B=3, len_lo=5, len_hi=40, k=16, H_I=4, H=2, w_std=0.5, seed=4)
    a = host_arrays(make_decode(cfg))
    res = oracle.decode(a)
    st = a["seq_start"]
    for r in res:
        b, Lb = r["seq"], r["L"]
        sl = slice(st[b], st[b + 1])
        if Lb <= 16:
            assert r["idx"].tolist() == list(range(Lb)) + [-1] * (16 - Lb)
        do, dl = oracle.dense_mla(a["q"][b:b + 1], a["kv"][sl], Lb - 1, a["sm_scale"])
        if Lb <= 16:
            assert np.allclose(r["out"], do[0], rtol=1e-12, atol=1e-13)
        # the decode query is the last row of a one-row prefill over its own cache
        sc = oracle.index_scores(a["q8"][b:b + 1], a["qs"][b:b + 1], a["w"][b:b + 1],
                                 a["k8"][sl], a["ks"][sl], Lb - 1, a["score_scale"])
        assert np.array_equal(sc[0], r["scores"])
        assert np.all(np.isfinite(r["scores"]))


# ----------------------------------------------------------------- fp8 input preparation

def _torch_quant(x: torch.Tensor):
    """The per-vector e4m3fn quantisation written with torch-CPU ops: fp32 amax / 448, fp32
    quotient, clamp (torch's cast does not saturate), torch's round-to-nearest-even cast."""
    amax = x.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (x / s.unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), s.numpy()


def test_quantize_matches_torch_cast_random_scales():
    g = torch.Generator().manual_seed(7)
    parts = []
    for mag in (1e-30, 1e-6, 1.0, 3.7, 1e4, 1e30):
        parts.append(torch.randn((64, 128), generator=g) * mag)
    x = torch.cat(parts)
    x[5, :] = 0.0                                     # all-zero vector: scale 1
    x[6, :] = -0.0                                    # negative zeros keep their sign
    x[7, :] = 0.0
    x[7, 9] = -2.5                                    # one non-zero element: it maps to -448
    q, s = oracle.quantize_e4m3(x.numpy())
    tq, ts = _torch_quant(x)
    assert np.array_equal(s, ts)
    assert np.array_equal(q, tq)
    assert s[5] == 1.0 and q[5].max() == 0 and np.all(q[6] == 0x80) and q[7, 9] == 0xFE


def test_quantize_ties_and_neighbours_match_torch_cast():
    """Scale exactly 1 (448 in every vector), the other entries every midpoint between
    adjacent e4m3fn values, those midpoints' fp32 neighbours, and the values themselves
    (both signs): the round-to-nearest-even rule, subnormals and the top of the range."""
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    mids = (vals[1:] + vals[:-1]) / 2                 # exact in fp32
    up = torch.nextafter(mids, torch.full_like(mids, 1e9))
    down = torch.nextafter(mids, torch.zeros_like(mids))
    pool = torch.cat([vals, mids, up, down, torch.tensor([2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11])])
    pool = torch.cat([pool, -pool])
    n = (len(pool) + 126) // 127
    x = torch.zeros((n, 128))
    flat = torch.cat([pool, torch.zeros(n * 127 - len(pool))])
    x[:, 1:] = flat.view(n, 127)
    x[:, 0] = 448.0
    q, s = oracle.quantize_e4m3(x.numpy())
    tq, ts = _torch_quant(x)
    assert np.all(s == 1.0) and np.array_equal(ts, s)
    assert np.array_equal(q, tq)


def test_quantize_bf16_input_matches_fp32_of_the_same_values():
    g = torch.Generator().manual_seed(3)
    xb = (torch.randn((50, 128), generator=g) * 5).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.quantize_e4m3(bits)
    tq, ts = _torch_quant(xb.to(torch.float32))
    assert np.array_equal(q, tq) and np.array_equal(s, ts)


def test_decode_append_writes_exactly_the_last_row_of_each_sequence():
    rng = np.random.default_rng(4)
    lens = np.array([3, 1, 7, 2])
    st = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = int(st[-1])
    k8 = rng.integers(0, 256, (N, 128), dtype=np.uint8)
    ks = rng.random(N).astype(np.float32)
    kv = rng.integers(0, 65536, (N, 576), dtype=np.uint16)
    k_new = rng.standard_normal((4, 128)).astype(np.float32)
    kv_new = rng.integers(0, 65536, (4, 576), dtype=np.uint16)
    k8_0, ks_0, kv_0 = k8.copy(), ks.copy(), kv.copy()
    oracle.decode_append(st, k_new, kv_new, k8, ks, kv)
    last = st[1:] - 1
    others = np.setdiff1d(np.arange(N), last)
    assert np.array_equal(k8[others], k8_0[others]) and np.array_equal(ks[others], ks_0[others])
    assert np.array_equal(kv[others], kv_0[others])
    tq, ts = _torch_quant(torch.from_numpy(k_new))
    assert np.array_equal(k8[last], tq) and np.array_equal(ks[last], ts)
    assert np.array_equal(kv[last], kv_new)


# ------------------------------------------------------------------ alternative index rules

def test_window_attention_matches_banded_sdpa():
    """Sliding-window attention as index lists: the sparse MLA over each row's window equals
    torch's attention with a band mask (tril/triu) of width W ending at the row's position."""
    a = _small_prefill(L=60, H=3, k=8, seed=17, q_pos0=10, T=50)
    T, L, W, q0 = 50, 60, 7, 10
    idx = oracle.window_indices(T, q0, W)
    out, lse = oracle.sparse_mla(a["q"], a["kv"], idx, 0.06)
    band = torch.ones((T, L), dtype=torch.bool).tril(q0).triu(q0 - W + 1)
    q = _deq16(a["q"]).permute(1, 0, 2).unsqueeze(0)
    kv = _deq16(a["kv"])
    K = kv.expand(3, L, 576).unsqueeze(0).contiguous()
    V = kv[:, :512].expand(3, L, 512).unsqueeze(0).contiguous()
    ro = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=band, scale=0.06)
    assert np.allclose(out, ro[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    # a window as long as the context is the dense causal attention
    full = oracle.window_indices(T, q0, L)
    fo, fl = oracle.sparse_mla(a["q"], a["kv"], full, 0.06)
    do, dl = oracle.dense_mla(a["q"], a["kv"], q0, 0.06)
    assert np.allclose(fo, do, rtol=1e-12, atol=1e-13) and np.allclose(fl, dl, rtol=1e-12)


def test_local_selected_is_the_sorted_union():
    rng = np.random.default_rng(9)
    T, k, W, q0 = 40, 6, 5, 20
    sel = np.full((T, k), -1, np.int32)
    for t in range(T):
        p = q0 + t
        m = int(rng.integers(0, k + 1))
        sel[t, :m] = np.sort(rng.choice(p + 1, size=m, replace=False))
    sel[3, 1] = -1                                    # a hole among the valid entries
    out = oracle.local_selected(sel, q0, W)
    assert out.shape == (T, W + k)
    for t in range(T):
        p = q0 + t
        win = torch.arange(max(0, p - W + 1), p + 1).numpy()
        want = np.union1d(win, sel[t][sel[t] >= 0])
        got = out[t]
        assert np.array_equal(got[:len(want)], want) and np.all(got[len(want):] == -1)
    # a window covering every visible position absorbs any selection
    wide = oracle.local_selected(sel, q0, q0 + T)
    for t in range(T):
        assert np.array_equal(wide[t][:q0 + t + 1], np.arange(q0 + t + 1))


# ------------------------------------------------------------------ packed (varlen) prefill

def _pack_full(seqs, lens_q, k):
    """A packed batch built from whole-sequence prefill inputs: sequence b keeps all its keys
    and its last lens_q[b] query rows."""
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum([s["L"] for s in seqs])]).astype(np.int64)
    pk = dict(k=k, cu_q=cu_q, cu_k=cu_k, score_scale=seqs[0]["score_scale"],
              sm_scale=seqs[0]["sm_scale"])
    for key in ("q8", "qs", "w", "q"):
        pk[key] = np.concatenate([s[key][s["T"] - t:] for s, t in zip(seqs, lens_q)])
    for key in ("k8", "ks", "kv"):
        pk[key] = np.concatenate([s[key] for s in seqs])
    return pk


def _full_seqs(lens_k, k, H_I, H, seed):
    return [host_arrays(make_prefill(PrefillCfg("t", L=L, k=k, H_I=H_I, H=H, w_std=0.5,
                                                seed=seed + b)))
            for b, L in enumerate(lens_k)]


def test_varlen_dense_equals_block_diagonal_sdpa():
    """Every sequence shorter than k: the packed batch is one attention over all packed
    tokens under a block-diagonal causal mask (query of sequence b at position
    L_b - T_b + t sees keys of sequence b at positions <= that), computed by torch."""
    lens_k, lens_q, k = [5, 3, 20, 7, 9], [5, 0, 12, 7, 1], 32
    pk = _pack_full(_full_seqs(lens_k, k, 4, 2, seed=70), lens_q, k)
    res = oracle.prefill_varlen(pk)
    assert res[1] is None
    for r in res:
        if r is not None:
            for t in range(r["T"]):
                n = r["q_pos0"] + t + 1
                assert r["idx"][t].tolist() == list(range(n)) + [-1] * (k - n)
    out = np.concatenate([r["out"] for r in res if r is not None])
    lse = np.concatenate([r["lse"] for r in res if r is not None])
    seq_q = np.repeat(np.arange(5), lens_q)
    pos_q = np.concatenate([np.arange(L - T, L) for T, L in zip(lens_q, lens_k)])
    seq_k = np.repeat(np.arange(5), lens_k)
    pos_k = np.concatenate([np.arange(L) for L in lens_k])
    mask = (seq_q[:, None] == seq_k[None, :]) & (pos_k[None, :] <= pos_q[:, None])
    q = _deq16(pk["q"]).permute(1, 0, 2).unsqueeze(0)
    kv = _deq16(pk["kv"])
    H, N = q.shape[1], kv.shape[0]
    K = kv.expand(H, N, 576).unsqueeze(0).contiguous()
    V = kv[:, :512].expand(H, N, 512).unsqueeze(0).contiguous()
    m = torch.from_numpy(mask)
    ro = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=m,
                                                          scale=pk["sm_scale"])
    rl = torch.logsumexp((q @ K.transpose(-1, -2) * pk["sm_scale"]).masked_fill(~m, -math.inf),
                         dim=-1)
    assert np.allclose(out, ro[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, rl[0].permute(1, 0).numpy(), rtol=1e-12, atol=1e-12)


def test_varlen_chunk_rows_equal_rows_of_the_whole_sequence_prefill():
    """Causality: a chunk of T_b new tokens prefilled against the cache of the first
    L_b - T_b tokens gives exactly the last T_b rows of prefilling the whole sequence
    (selection included, with k well below L_b)."""
    lens_k, lens_q, k = [30, 40, 6, 25, 64], [30, 11, 0, 1, 33], 8
    seqs = _full_seqs(lens_k, k, 4, 3, seed=80)
    res = oracle.prefill_varlen(_pack_full(seqs, lens_q, k))
    for b, (s, T) in enumerate(zip(seqs, lens_q)):
        if T == 0:
            assert res[b] is None
            continue
        full = oracle.prefill(s)
        L = s["L"]
        assert np.array_equal(res[b]["idx"], full["idx"][L - T:])
        assert np.array_equal(res[b]["n_vis"], full["n_vis"][L - T:])
        assert np.allclose(res[b]["scores"], full["scores"][L - T:], rtol=0, atol=0)
        assert np.allclose(res[b]["out"], full["out"][L - T:], rtol=1e-14, atol=1e-15)
        assert np.allclose(res[b]["lse"], full["lse"][L - T:], rtol=1e-14, atol=1e-15)


def test_varlen_sequences_are_isolated_and_order_free():
    """Reordering the sequences, or changing one sequence's keys, leaves every other
    sequence's result unchanged."""
    lens_k, lens_q, k = [26, 50, 19], [26, 20, 7], 6
    seqs = _full_seqs(lens_k, k, 2, 2, seed=90)
    base = oracle.prefill_varlen(_pack_full(seqs, lens_q, k))
    order = [2, 0, 1]
    perm = oracle.prefill_varlen(_pack_full([seqs[i] for i in order],
                                            [lens_q[i] for i in order], k))
    for j, i in enumerate(order):
        for key in ("idx", "out", "lse"):
            assert np.array_equal(perm[j][key], base[i][key])
    changed = [dict(s) for s in seqs]
    changed[1]["kv"] = changed[1]["kv"][::-1].copy()
    changed[1]["k8"] = changed[1]["k8"][::-1].copy()
    alt = oracle.prefill_varlen(_pack_full(changed, lens_q, k))
    assert not np.array_equal(alt[1]["out"], base[1]["out"])
    for i in (0, 2):
        for key in ("idx", "out", "lse"):
            assert np.array_equal(alt[i][key], base[i][key])


# ------------------------------------------------------------------ indexer warm-up (KL)

def _torch_warmup(x):
    """The warm-up loss written with torch float64 library ops, differentiated by autograd."""
    QI = torch.tensor(x["QI"], requires_grad=True)
    KI = torch.tensor(x["KI"], requires_grad=True)
    w = torch.tensor(x["w"], requires_grad=True)
    q, kv = torch.tensor(x["q"]), torch.tensor(x["kv"])
    pos = torch.tensor(x["pos"])
    L = KI.shape[0]
    vis = torch.arange(L)[None, :] <= pos[:, None]                       # [n, L]
    logits = torch.einsum("nhd,sd->nhs", q, kv) * x["sm_scale"]
    logits = logits.masked_fill(~vis[:, None, :], -math.inf)
    P = torch.softmax(logits, dim=-1).mean(dim=1)                        # head average
    I = x["c"] * (w[:, :, None] * torch.relu(torch.einsum("nhd,sd->nhs", QI, KI))).sum(1)
    logQ = torch.log_softmax(I.masked_fill(~vis, -math.inf), dim=-1).masked_fill(~vis, 0.0)
    kl = torch.nn.functional.kl_div(logQ, P, reduction="none").sum(-1)
    kl.sum().backward()
    G = (torch.exp(logQ) * vis - P).detach()
    return dict(kl=kl.detach().numpy(), P=P.detach().numpy(), G=G.numpy(),
                lse_t=torch.logsumexp(logits, -1).detach().numpy(),
                lse_i=torch.logsumexp(I.masked_fill(~vis, -math.inf), -1).detach().numpy(),
                dq=QI.grad.numpy(), dk=KI.grad.numpy(), dw=w.grad.numpy())


@pytest.mark.parametrize("L,T,q_pos0,H_I,H,seed", [(40, 40, 0, 3, 4, 1), (57, 30, 27, 4, 2, 2),
                                                    (33, 33, 0, 1, 3, 3)])
def test_warmup_matches_torch_autograd(L, T, q_pos0, H_I, H, seed):
    a = host_arrays(make_prefill(PrefillCfg("t", L=L, k=8, H_I=H_I, H=H, w_std=0.7, seed=seed,
                                            q_pos0=q_pos0, T=T)))
    x = oracle.warmup_inputs(a)
    o = oracle.warmup(x, want_dk=True, dist=True)
    ref = _torch_warmup(x)
    for key in ("kl", "P", "G", "lse_t", "lse_i", "dq", "dk", "dw"):
        scale = np.abs(ref[key]).max()
        assert np.allclose(o[key], ref[key], rtol=1e-9, atol=1e-12 * max(scale, 1.0)), key


def test_warmup_homogeneity_identities_and_bounds():
    """The scores are homogeneous of degree one in w, in each query vector and in each key
    vector, so <dw, w> = <dq, QI> = sum_s G I per row, and <dk, KI> is their sum over rows;
    every bound dominates its value."""
    a = host_arrays(make_prefill(PrefillCfg("t", L=50, k=8, H_I=4, H=3, w_std=0.7, seed=7)))
    x = oracle.warmup_inputs(a)
    o = oracle.warmup(x, want_dk=True, dist=True, bounds=True)
    xv = np.einsum("nhd,sd->nhs", x["QI"], x["KI"])
    I = x["c"] * (x["w"][:, :, None] * np.maximum(xv, 0)).sum(1)
    vis = np.arange(50)[None, :] <= x["pos"][:, None]
    gi = (o["G"] * np.where(vis, I, 0)).sum(1)
    assert np.allclose((o["dw"] * x["w"]).sum(1), gi, rtol=1e-10, atol=1e-14)
    assert np.allclose((o["dq"] * x["QI"]).sum((1, 2)), gi, rtol=1e-10, atol=1e-14)
    assert np.isclose((o["dk"] * x["KI"]).sum(), gi.sum(), rtol=1e-10, atol=1e-14)
    assert np.allclose(o["P"].sum(1), 1.0, rtol=1e-13) and np.allclose(o["G"].sum(1), 0, atol=1e-14)
    assert (o["kl"] >= -1e-15).all() and (o["kl_bnd"] >= np.abs(o["kl"])).all()
    assert (o["dw_bnd"] >= np.abs(o["dw"]) - 1e-15).all()
    assert (o["dq_bnd"] >= np.abs(o["dq"]) - 1e-15).all()
    assert (o["dk_bnd"] >= np.abs(o["dk"]) - 1e-15).all()


def _exact_warmup_inputs(L, T, q_pos0, H_I, H, seed, planted):
    """Warm-up inputs whose indexer dot products are exact in any summation order: query and
    key vectors are e4m3 values times powers of two (products have at most 8 significant bits,
    sums stay far inside fp64's 53).  `planted` (row, head, key) triples get a key that is the
    query vector rotated pairwise, (a, b) -> (b, -a), so their dot product is exactly zero while
    the sum of |products| is not: the terms whose ReLU decision a rounded dot may flip."""
    g = torch.Generator().manual_seed(seed)
    def e4(shape, exps):
        v = (torch.randn(shape, generator=g) * 3).to(torch.float8_e4m3fn).to(torch.float64)
        return v * (2.0 ** exps)
    QI = e4((T, H_I, 128), torch.randint(-3, 3, (T, H_I, 1), generator=g).double())
    KI = e4((L, 128), torch.randint(-2, 2, (L, 1), generator=g).double())
    for r, h, s in planted:
        v = QI[r, h]
        rot = torch.stack([v[1::2], -v[0::2]], dim=1).reshape(128)
        KI[s] = rot
    w = torch.randn((T, H_I), generator=g, dtype=torch.float64) * 0.7
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16).double()
    kv = torch.randn((L, 576), generator=g).to(torch.bfloat16).double()
    return dict(QI=QI.numpy(), KI=KI.numpy(), w=w.numpy(), q=q.numpy(), kv=kv.numpy(),
                pos=q_pos0 + np.arange(T), c=0.125, sm_scale=576 ** -0.5)


def _tolerance_terms(x, P, logQ):
    """The warm-up's tolerance ingredients from their definitions, vectorised in numpy, with
    the target P and log Q taken from the torch autograd reference: A = Q + P (the magnitude
    that stands in for |G| = |Q - P|), x = <QI, KI> per (row, head, key), |x|_1 = sum_d |QI KI|,
    a term ambiguous when |x| <= 2^-16 |x|_1 (a rounded dot may land on either side of 0)."""
    QI, KI, w, c = x["QI"], x["KI"], x["w"], x["c"]
    L = KI.shape[0]
    vis = np.arange(L)[None, :] <= x["pos"][:, None]                     # [n, L]
    Q = np.where(vis, np.exp(logQ), 0.0)
    A = np.where(vis, Q + P, 0.0)
    xv = np.einsum("nhd,sd->nhs", QI, KI)
    xa = np.einsum("nhd,sd->nhs", np.abs(QI), np.abs(KI))
    pos_ = (xv > 0) & vis[:, None, :]
    amb = (np.abs(xv) <= 2.0 ** -16 * xa) & vis[:, None, :]
    cw = np.abs(c * w)                                                   # [n, H_I]
    t = dict(amb_count=int(amb.sum()))
    t["dq_bnd"] = cw[:, :, None] * np.einsum("nhs,ns,sd->nhd", pos_.astype(float), A, np.abs(KI))
    t["dq_amb"] = cw[:, :, None] * np.einsum("nhs,ns,sd->nhd", amb.astype(float), A, np.abs(KI))
    t["dk_bnd"] = np.einsum("nhs,nh,ns,nhd->sd", pos_.astype(float), cw, A, np.abs(QI))
    t["dk_amb"] = np.einsum("nhs,nh,ns,nhd->sd", amb.astype(float), cw, A, np.abs(QI))
    t["dw_bnd"] = abs(c) * np.einsum("ns,nhs->nh", A, np.abs(xv) * vis[:, None, :])
    with np.errstate(divide="ignore", invalid="ignore"):
        lp = np.where(P > 0, np.log(np.where(P > 0, P, 1.0)), 0.0)
    t["kl_bnd"] = (np.where(P > 0, P * (np.abs(lp) + np.abs(np.where(vis, logQ, 0.0))), 0.0)).sum(1)
    return t


@pytest.mark.parametrize("L,T,q_pos0,H_I,H,seed", [(50, 50, 0, 4, 3, 21), (40, 25, 15, 64, 2, 22)])
def test_warmup_tolerance_terms_equal_their_definitions(L, T, q_pos0, H_I, H, seed):
    """Every tolerance ingredient of the warm-up parity check (dq/dk ambiguity sums and the
    dq/dk/dw/kl magnitude sums) equals an independent numpy evaluation of its definition, on
    inputs with planted exactly-cancelling (row, head, key) terms.  An ambiguity sum that
    counted every term, or a magnitude sum over all keys instead of the ReLU-active ones,
    fails here; so does a dropped |w| or a missing Q + P weight."""
    planted = [(3, 1, 2), (7, 0, 5), (T - 1, H_I - 1, q_pos0 + T - 2), (10, 2, 9)]
    x = _exact_warmup_inputs(L, T, q_pos0, H_I, H, seed, planted)
    o = oracle.warmup(x, want_dk=True, dist=True, bounds=True)
    ref = _torch_warmup(x)
    # log Q = I - lse_i, with the student scores I from exact dots and lse_i from torch
    I = x["c"] * np.einsum("nh,nhs->ns", x["w"], np.maximum(
        np.einsum("nhd,sd->nhs", x["QI"], x["KI"]), 0.0))
    vis = np.arange(L)[None, :] <= x["pos"][:, None]
    logQ = np.where(vis, I - ref["lse_i"][:, None], 0.0)
    t = _tolerance_terms(x, ref["P"], logQ)
    assert t["amb_count"] >= len(planted)          # the plant is seen as ambiguous
    for key in ("dq_bnd", "dq_amb", "dk_bnd", "dk_amb", "dw_bnd", "kl_bnd"):
        scale = max(np.abs(t[key]).max(), 1e-300)
        assert np.allclose(o[key], t[key], rtol=1e-11, atol=1e-13 * scale), key
    # the ambiguity sums are nonzero exactly where a planted term sits, and zero elsewhere
    for r, h, s in planted:
        assert (o["dq_amb"][r, h] > 0).any() and (o["dk_amb"][s] > 0).any()
    amb_rows = {(r, h) for r, h, _ in planted}
    for r in range(T):
        for h in range(H_I):
            if (r, h) not in amb_rows and t["dq_amb"][r, h].max() == 0:
                assert o["dq_amb"][r, h].max() == 0.0


def test_warmup_ambiguity_sums_vanish_without_near_zero_dots():
    """On inputs with no planted cancellation every (row, head, key) dot product is far from
    zero relative to its |products| sum (checked in numpy), so the ambiguity sums are exactly
    zero: they cannot widen the dq/dk tolerance when no ReLU decision is in doubt."""
    x = _exact_warmup_inputs(45, 45, 0, 4, 2, 23, planted=[])
    xv = np.einsum("nhd,sd->nhs", x["QI"], x["KI"])
    xa = np.einsum("nhd,sd->nhs", np.abs(x["QI"]), np.abs(x["KI"]))
    vis = np.arange(45)[None, None, :] <= x["pos"][:, None, None]
    assert not ((np.abs(xv) <= 2.0 ** -16 * xa) & vis).any()
    o = oracle.warmup(x, want_dk=True, bounds=True)
    assert np.all(o["dq_amb"] == 0.0) and np.all(o["dk_amb"] == 0.0)


def test_warmup_student_equal_to_teacher_has_zero_loss():
    """When the indexer's distribution is the target itself the loss and every gradient
    vanish: one indexer head with QI = e_0, KI[s] = log-target in dimension 0 (positive
    part only is kept by the ReLU, so the target is made of positive log-ratios), w = 1/c."""
    L = 6
    rng = np.random.default_rng(3)
    target = rng.uniform(1.0, 3.0, L)                 # I[s] for the last row
    x = dict(QI=np.zeros((1, 1, 128)), w=np.array([[1.0 / 0.25]]), KI=np.zeros((L, 128)),
             q=np.zeros((1, 2, 576)), kv=np.zeros((L, 576)), pos=np.array([L - 1]), c=0.25,
             sm_scale=0.1)
    x["QI"][0, 0, 0] = 1.0
    x["KI"][:, 0] = target
    # teacher logits sm_scale <q_h, kv_s> = target[s] for both heads: q_h = e_0 / sm_scale
    x["q"][0, :, 0] = 1.0 / 0.1
    x["kv"][:, 0] = target
    o = oracle.warmup(x, want_dk=True, dist=True)
    assert abs(o["kl"][0]) < 1e-14
    assert np.abs(o["G"]).max() < 1e-15
    assert np.abs(o["dq"]).max() < 1e-13 and np.abs(o["dk"]).max() < 1e-13
    assert np.abs(o["dw"]).max() < 1e-13
