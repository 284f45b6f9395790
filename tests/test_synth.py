"""The seeded input generator: determinism, the storage formats, the planted tokens."""
import hashlib

import numpy as np
import torch

from synth import DecodeCfg, PrefillCfg, host_arrays, make_decode, make_prefill, quantize_e4m3_rows


def _digest(a: dict) -> str:
    h = hashlib.sha256()
    for key in ("q8", "qs", "w", "k8", "ks", "q", "kv"):
        h.update(np.ascontiguousarray(a[key]).tobytes())
    return h.hexdigest()


def test_prefill_is_deterministic_per_seed():
    cfg = PrefillCfg("t", L=64, k=16, H_I=4, H=2, w_std=0.5, seed=3, planted_frac=0.05)
    a, b = host_arrays(make_prefill(cfg)), host_arrays(make_prefill(cfg))
    c = host_arrays(make_prefill(cfg, seed=4))
    assert _digest(a) == _digest(b) != _digest(c)
    assert a["q8"].shape == (64, 4, 128) and a["kv"].shape == (64, 576)


def test_e4m3_quantisation_rows():
    g = torch.Generator().manual_seed(0)
    v = torch.randn((200, 128), generator=g) * torch.logspace(-3, 3, 200).unsqueeze(1)
    v[7] = 0.0
    code, scale = quantize_e4m3_rows(v)
    deq = code.view(torch.float8_e4m3fn).to(torch.float64)
    assert torch.all(scale[7] == 1.0) and torch.all(code[7] == 0)
    nz = torch.arange(200) != 7
    # the largest magnitude of each row lands on the largest finite code
    assert torch.all(deq[nz].abs().amax(1) == 448.0)
    rel = (deq * scale.double().unsqueeze(1) - v.double()).abs()
    x = (v.double() / scale.double().unsqueeze(1)).abs()
    normal = x >= 2 ** -6
    assert torch.all(rel[normal] <= 2 ** -4 * v.double().abs()[normal] * (1 + 1e-6))
    assert torch.all(rel[~normal] <= 2 ** -10 * scale.double().unsqueeze(1).expand_as(rel)[~normal] * (1 + 1e-6))
    assert not torch.isnan(deq).any()


def test_planted_keys_point_at_their_target_query_head():
    cfg = PrefillCfg("t", L=400, k=64, H_I=8, H=2, w_std=1 / 8 ** 0.5, seed=5, planted_frac=0.01)
    a = host_arrays(make_prefill(cfg))
    pl = a["planted"]
    assert len(pl) == 4
    deq = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    for s, t, h in pl:
        assert max(s, cfg.k) <= t < cfg.L
        assert h == np.argmax(a["w"][t])
        kv, qv = deq(a["k8"][s]), deq(a["q8"][t, h])
        cos = kv @ qv / np.linalg.norm(kv) / np.linalg.norm(qv)
        assert cos > 0.98


def test_decode_lengths_and_packing():
    cfg = DecodeCfg("t", B=6, len_lo=10, len_hi=50, k=8, H_I=4, H=2, w_std=0.5, seed=1)
    a = host_arrays(make_decode(cfg))
    lens = np.diff(a["seq_start"])
    assert np.all((lens >= 10) & (lens <= 50))
    assert a["seq_start"][0] == 0 and a["seq_start"][-1] == a["N"] == a["k8"].shape[0]
    assert a["kv"].shape == (a["N"], 576) and a["q"].shape == (6, 2, 576)


def test_varlen_lengths_and_packing():
    from synth import WORKLOADS, make_varlen
    cfg = WORKLOADS["varlen-B16-L1024-32768-k2048"]
    T, L = cfg.lengths()
    assert (T, L) == cfg.lengths() and len(T) == len(L) == cfg.B
    for b, (t, l) in enumerate(zip(T, L)):
        assert cfg.len_lo <= l <= cfg.len_hi
        assert t == l if b % 2 == 0 else min(cfg.chunk_lo, l) <= t <= min(cfg.chunk_hi, l)
    a = make_varlen([3, 0, 5], [4, 2, 5], k=4, H_I=2, H=2, w_std=0.5, seed=1)
    b = make_varlen([3, 0, 5], [4, 2, 5], k=4, H_I=2, H=2, w_std=0.5, seed=1)
    assert a["cu_q"].tolist() == [0, 3, 3, 8] and a["cu_k"].tolist() == [0, 4, 6, 11]
    assert a["q8"].shape == (8, 2, 128) and a["kv"].shape == (11, 576)
    for key in ("q8", "qs", "w", "q", "k8", "ks", "kv"):
        assert torch.equal(a[key], b[key])
    # each sequence is the prefill workload of its own seed: its last T_b query rows
    one = make_prefill(PrefillCfg("varlen-seq2", L=5, k=4, H_I=2, H=2, w_std=0.5,
                                  seed=1 * 1009 + 2, T=5))
    assert torch.equal(a["q"][3:8], one["q"]) and torch.equal(a["kv"][6:11], one["kv"])
