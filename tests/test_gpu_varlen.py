"""Packed (varlen) prefill on the HIP path vs the CPU oracle, through the C ABI (needs an
MI355X).

A batch of B sequences packed by host cu_seqlens: sequence b's T_b queries are its last T_b
tokens (fresh prefill when T_b = L_b, a chunk against a cache otherwise).  Small ragged
batches compare every row; the 16-sequence serving batch runs in the benchmark's launch
configuration and compares sampled rows of every sequence.  Tolerances: tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import check_indices_near_ties, check_mla, bf16_to_f64, oracle_prefill_rows
from synth import WORKLOADS, host_arrays, make_varlen, make_varlen_cfg

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(dsa, d, with_idx=True):
    idx = (torch.full((d["Tq"], d["k"]), -7, dtype=torch.int32, device="cuda")
           if with_idx else None)
    out, lse, _ = dsa.dsa_prefill_varlen(d["cu_q"], d["cu_k"], d["q8"], d["qs"], d["w"],
                                         d["k8"], d["ks"], d["q"], d["kv"], d["k"],
                                         d["score_scale"], d["sm_scale"], idx_out=idx)
    torch.cuda.synchronize()
    return out, lse, idx


def _seq(d, b):
    """Sequence b of a packed device batch as a single prefill call's inputs."""
    qa, qe = int(d["cu_q"][b]), int(d["cu_q"][b + 1])
    ka, ke = int(d["cu_k"][b]), int(d["cu_k"][b + 1])
    s = dict(T=qe - qa, L=ke - ka, q_pos0=(ke - ka) - (qe - qa), k=d["k"],
             score_scale=d["score_scale"], sm_scale=d["sm_scale"], qa=qa, qe=qe)
    for key in ("q8", "qs", "w", "q"):
        s[key] = d[key][qa:qe]
    for key in ("k8", "ks", "kv"):
        s[key] = d[key][ka:ke]
    return s


# ragged lengths: an empty query set over a cache, a 1-token sequence, fresh prefills just
# above / at / below k, chunks against caches, a chunk of one token
SMALL = dict(lens_q=[0, 1, 300, 137, 64, 500, 3, 1, 257],
             lens_k=[5, 1, 300, 900, 64, 1300, 3, 777, 257])


@pytest.mark.parametrize("H_I,H,k", [(64, 16, 256), (4, 8, 64)])
def test_varlen_small_every_row(dsa, H_I, H, k):
    d = make_varlen(SMALL["lens_q"], SMALL["lens_k"], k=k, H_I=H_I, H=H, w_std=H_I ** -0.5,
                    seed=31, device="cuda")
    out, lse, idx = _run(dsa, d)
    gidx = _np(idx)
    assert (gidx != -7).all()
    h = host_arrays(d)
    ref = oracle.prefill_varlen(h, with_bound=True)
    for b, r in enumerate(ref):
        s = _seq(d, b)
        if r is None:
            assert s["T"] == 0
            continue
        sl = slice(s["qa"], s["qe"])
        what = "varlen seq %d (T=%d, L=%d)" % (b, s["T"], s["L"])
        check_indices_near_ties(gidx[sl], r["idx"], r["scores"], r["bound"], r["n_vis"], k,
                                what)
        oo, ol = oracle.sparse_mla(_u16(s["q"]), _u16(s["kv"]), gidx[sl], s["sm_scale"])
        check_mla(bf16_to_f64(out[sl]), _np(lse[sl]), oo, ol, what)


def test_varlen_equals_per_sequence_prefill_bitwise(dsa):
    """The packed call computes each sequence exactly as dsa_prefill with q_pos0 = L_b - T_b."""
    d = make_varlen(SMALL["lens_q"], SMALL["lens_k"], k=128, H_I=64, H=32, w_std=1 / 8,
                    seed=32, device="cuda")
    out, lse, idx = _run(dsa, d)
    for b in range(len(SMALL["lens_q"])):
        s = _seq(d, b)
        if s["T"] == 0:
            continue
        one_idx = torch.empty((s["T"], 128), dtype=torch.int32, device="cuda")
        o, l, _ = dsa.dsa_prefill(s["q8"], s["qs"], s["w"], s["k8"], s["ks"], s["q"], s["kv"],
                                  128, s["q_pos0"], s["score_scale"], s["sm_scale"],
                                  idx_out=one_idx)
        torch.cuda.synchronize()
        sl = slice(s["qa"], s["qe"])
        assert torch.equal(one_idx, idx[sl]), "seq %d indices" % b
        assert torch.equal(o, out[sl]) and torch.equal(l, lse[sl]), "seq %d output" % b


def test_varlen_short_sequences_are_block_diagonal_dense_attention(dsa):
    """Every sequence within k tokens: selection is everything visible, and each row is
    exact causal attention over its own sequence."""
    lens_k = [1, 2, 17, 64, 200, 511, 512]
    lens_q = [1, 1, 17, 10, 200, 1, 300]
    d = make_varlen(lens_q, lens_k, k=512, H_I=8, H=16, w_std=0.35, seed=33, device="cuda")
    out, lse, idx = _run(dsa, d)
    gidx = _np(idx)
    for b in range(len(lens_k)):
        s = _seq(d, b)
        sl = slice(s["qa"], s["qe"])
        p = s["q_pos0"] + np.arange(s["T"])
        want = np.where(np.arange(512)[None, :] <= p[:, None], np.arange(512)[None, :], -1)
        assert np.array_equal(gidx[sl], want), "seq %d" % b
        do, dl = oracle.dense_mla(_u16(s["q"]), _u16(s["kv"]), s["q_pos0"], s["sm_scale"])
        check_mla(bf16_to_f64(out[sl]), _np(lse[sl]), do, dl, "dense seq %d" % b)


def test_varlen_empty_batches_are_no_ops(dsa):
    d = make_varlen([0, 0], [3, 9], k=64, H_I=4, H=8, w_std=0.5, seed=34, device="cuda")
    out, lse, idx = _run(dsa, d)
    assert out.shape == (0, 8, 512) and idx.shape == (0, 64)
    z = make_varlen([], [], k=64, H_I=4, H=8, w_std=0.5, seed=34, device="cuda")
    out, lse, idx = _run(dsa, z)
    assert out.shape == (0, 8, 512)


def test_varlen_idx_out_optional_and_repeatable(dsa):
    d = make_varlen([300, 99, 450], [300, 700, 451], k=96, H_I=64, H=16, w_std=1 / 8,
                    seed=35, device="cuda")
    o1, l1, _ = _run(dsa, d, with_idx=False)
    o2, l2, i2 = _run(dsa, d)
    o3, l3, i3 = _run(dsa, d)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o2, o3) and torch.equal(l2, l3) and torch.equal(i2, i3)


def test_varlen_serving_batch_sampled_rows(dsa):
    """16 sequences of 1K..32K tokens, every other one a chunk against a cache, in the
    benchmark's launch configuration; sampled rows of every sequence against the oracle."""
    cfg = WORKLOADS["varlen-B16-L1024-32768-k2048"]
    d = make_varlen_cfg(cfg, device="cuda")
    out, lse, idx = _run(dsa, d)
    rng = np.random.default_rng(cfg.seed)
    checked = 0
    for b in range(cfg.B):
        s = _seq(d, b)
        T, k = s["T"], cfg.k
        first_sel = max(0, k - s["q_pos0"])             # first row that sees more than k
        fixed = [0, T - 1, min(T - 1, first_sel), min(T - 1, first_sel + 1)]
        rows = np.unique(np.array(fixed + rng.integers(0, T, 2).tolist()))
        sel = torch.from_numpy(rows + s["qa"]).cuda()
        gidx, go, gl = _np(idx[sel]), out[sel], lse[sel]
        ora = oracle_prefill_rows(s, rows, k)
        kv = _u16(s["kv"])
        for i, r in enumerate(ora):
            what = "varlen seq %d row %d (T=%d, L=%d)" % (b, r["t"], T, s["L"])
            check_indices_near_ties(gidx[i:i + 1], r["idx"][None], r["scores"][None],
                                    r["bound"][None], [r["n"]], k, what)
            oo, ol = oracle.sparse_mla(_u16(s["q"][r["t"]:r["t"] + 1]), kv, gidx[i:i + 1],
                                       s["sm_scale"])
            check_mla(bf16_to_f64(go[i:i + 1]), _np(gl[i:i + 1]), oo, ol, what)
            checked += 1
    assert checked >= 3 * cfg.B
