"""Seeded random small shapes through the fused prefill, the decode step and the indexer
warm-up, against the CPU oracle (needs an MI355X): odd and tiny T, L, q_pos0, k and head
counts, including the degenerate ones (one key, one query row, k = 1, k >= L), and decode
batches whose lengths straddle the top-k's whole-row staging limit and its 16K-key segments.
Tolerances: tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle
from parity import (bf16_to_f64, check_decode, check_indices_near_ties, check_mla,
                    check_warmup_dk, check_warmup_rows)
from synth import DecodeCfg, PrefillCfg, host_arrays, make_decode, make_prefill

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _shapes(seed, n, k_choices, hi_choices, h_choices, l_max):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        L = int(rng.integers(1, l_max + 1))
        T = int(rng.integers(1, L + 1))
        q0 = int(rng.integers(0, L - T + 1))
        out.append((L, T, q0, int(rng.choice(k_choices)), int(rng.choice(hi_choices)),
                    int(rng.choice(h_choices)), 100 + i))
    # the degenerate corners
    out += [(1, 1, 0, 1, hi_choices[0], 1, 90), (5, 1, 4, 1, hi_choices[-1], 3, 91),
            (37, 37, 0, 64, hi_choices[0], 5, 92)]
    return out


@pytest.mark.parametrize("L,T,q0,k,H_I,H,seed",
                         _shapes(7, 10, [1, 2, 7, 64, 255, 2048], [4, 16, 64], [1, 7, 16, 40],
                                 900))
def test_prefill_random_shape(dsa, L, T, q0, k, H_I, H, seed):
    cfg = PrefillCfg("rand", L=L, k=k, H_I=H_I, H=H, w_std=H_I ** -0.5, seed=seed, q_pos0=q0,
                     T=T)
    inp = make_prefill(cfg)
    h = host_arrays(inp)
    d = {key: (v.cuda() if isinstance(v, torch.Tensor) else v) for key, v in inp.items()}
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_prefill(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                  k, q0, cfg.score_scale, cfg.sm_scale, idx_out=idx)
    torch.cuda.synchronize()
    ref = oracle.prefill(h, with_bound=True)
    gidx = _np(idx)
    what = "prefill L=%d T=%d q_pos0=%d k=%d H_I=%d H=%d" % (L, T, q0, k, H_I, H)
    check_indices_near_ties(gidx, ref["idx"], ref["scores"], ref["bound"], ref["n_vis"], k, what)
    n = np.minimum(q0 + np.arange(T) + 1, k)
    assert all((gidx[t, n[t]:] == -1).all() for t in range(T)), what + ": padding"
    oo, ol = oracle.sparse_mla(h["q"], h["kv"], gidx, cfg.sm_scale)
    check_mla(bf16_to_f64(out), _np(lse), oo, ol, what)


@pytest.mark.parametrize("L,T,q0,k,H_I,H,seed",
                         _shapes(11, 6, [0], [16, 32, 64, 128], [1, 3, 16, 33, 128], 420))
def test_warmup_random_shape(dsa, L, T, q0, k, H_I, H, seed):
    cfg = PrefillCfg("rand", L=L, k=8, H_I=H_I, H=H, w_std=H_I ** -0.5, seed=seed, q_pos0=q0,
                     T=T)
    d = make_prefill(cfg, device="cuda")
    res = dsa.dsa_indexer_warmup(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                 q0, cfg.score_scale, cfg.sm_scale)
    torch.cuda.synchronize()
    g = {key: _np(v) for key, v in res.items()}
    x = oracle.warmup_inputs(host_arrays({key: d[key] for key in
                                          ("q8", "qs", "w", "q", "k8", "ks", "kv")} |
                                         dict(q_pos0=q0, score_scale=cfg.score_scale,
                                              sm_scale=cfg.sm_scale)))
    o = oracle.warmup(x, want_dk=True, bounds=True)
    what = "warm-up L=%d T=%d q_pos0=%d H_I=%d H=%d" % (L, T, q0, H_I, H)
    check_warmup_rows(g, o, np.arange(T), what)
    check_warmup_dk(g["dk"], o, what)


def _decode_shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        lo = int(rng.integers(1, 20001))
        hi = lo + int(rng.integers(0, 20001))
        H_I = int(rng.choice([1, 8, 32, 64, 128]))
        out.append((int(rng.integers(1, 7)), lo, hi, int(rng.choice([1, 7, 64, 255, 2048, 8192])),
                    H_I, int(rng.choice([1, 7, 16, 128])), 300 + i))
    # one token; lengths within k; around the staging limit and a segment boundary
    out += [(1, 1, 1, 1, 64, 8, 290), (3, 1, 3, 2048, 4, 16, 291),
            (4, 5880, 5896, 2048, 64, 16, 292), (3, 16380, 16390, 2048, 16, 8, 293)]
    return out


@pytest.mark.parametrize("B,lo,hi,k,H_I,H,seed", _decode_shapes(13, 6))
def test_decode_random_shape(dsa, B, lo, hi, k, H_I, H, seed):
    cfg = DecodeCfg("rand", B=B, len_lo=lo, len_hi=hi, k=k, H_I=H_I, H=H, w_std=H_I ** -0.5,
                    seed=seed)
    inp = make_decode(cfg)
    check_decode(dsa, inp, range(B), "decode B=%d L=[%d,%d] k=%d H_I=%d H=%d" % (
        B, lo, hi, k, H_I, H))
