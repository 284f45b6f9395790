"""Alternative index rules (sliding window, local + selected) feeding the sparse MLA: HIP path
vs the CPU oracle through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from parity import bf16_to_f64, check_mla, to_device
from synth import PrefillCfg, host_arrays, make_prefill

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,L,q0,W", [(1, 1, 0, 1), (300, 300, 0, 64), (77, 5000, 4923, 2048),
                                      (130, 200, 70, 500), (64, 64, 0, 1)])
def test_window_indices_match_oracle(dsa, T, L, q0, W):
    idx = dsa.dsa_window_indices(T, L, q0, W)
    torch.cuda.synchronize()
    assert np.array_equal(_np(idx), oracle.window_indices(T, q0, W))


def test_local_selected_on_topk_output_matches_oracle(dsa):
    cfg = PrefillCfg("c", L=3000, k=256, H_I=4, H=8, w_std=0.5, seed=31, T=900, q_pos0=2100)
    d = to_device(make_prefill(cfg))
    sc = dsa.dsa_index_scores(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], cfg.q_pos0,
                              cfg.score_scale)
    sel = dsa.dsa_topk(sc, cfg.L, cfg.q_pos0, cfg.k)
    sel[5, 7] = -1                                    # holes among the valid entries
    sel[6, ::3] = -1
    for W in (1, 64, 3000):
        out = dsa.dsa_local_selected_indices(sel, cfg.L, cfg.q_pos0, W)
        torch.cuda.synchronize()
        assert np.array_equal(_np(out), oracle.local_selected(_np(sel), cfg.q_pos0, W)), W


@pytest.mark.parametrize("W", [16, 200])
def test_window_attention_matches_oracle(dsa, W):
    cfg = PrefillCfg("c", L=700, k=64, H_I=4, H=16, w_std=0.5, seed=41, T=400, q_pos0=300)
    inp = make_prefill(cfg)
    h, d = host_arrays(inp), to_device(inp)
    idx = dsa.dsa_window_indices(cfg.T, cfg.L, cfg.q_pos0, W)
    out, lse = dsa.dsa_sparse_mla(d["q"], d["kv"], idx, cfg.sm_scale)
    torch.cuda.synchronize()
    oo, ol = oracle.sparse_mla(h["q"], h["kv"], oracle.window_indices(cfg.T, cfg.q_pos0, W),
                               cfg.sm_scale)
    check_mla(bf16_to_f64(out), _np(lse), oo, ol, "window %d" % W)


def test_window_attention_128k_sampled_rows(dsa):
    """Window 2048 over the 128K workload in the benchmark's launch configuration (the prefill's
    query chunks: the window lists, then the sparse MLA on them); sampled rows of the launched chunks
    against the oracle, indices exactly."""
    from synth import WORKLOADS
    cfg = WORKLOADS["prefill-L131072-k2048"]
    W, chunk = 2048, dsa.dsa_prefill_chunk_rows(cfg.L, cfg.L)
    d = make_prefill(cfg, device="cuda")
    kv = _u16(d["kv"])
    rows = np.array([0, 1, W - 2, W - 1, W, W + 1, 65535, 65536, 100001, cfg.L - 1])
    idx = torch.empty((chunk, W), dtype=torch.int32, device="cuda")
    for c in sorted(set((rows // chunk).tolist())):
        r0 = c * chunk
        r1 = min(cfg.L, r0 + chunk)
        ic = idx[:r1 - r0]
        dsa.dsa_window_indices(r1 - r0, cfg.L, r0, W, idx=ic)
        out, lse = dsa.dsa_sparse_mla(d["q"][r0:r1], d["kv"], ic, cfg.sm_scale)
        torch.cuda.synchronize()
        for t in rows[(rows >= r0) & (rows < r1)]:
            i = int(t) - r0
            want = oracle.window_indices(1, int(t), W)
            assert np.array_equal(_np(ic[i:i + 1]), want), "window row %d" % t
            oo, ol = oracle.sparse_mla(_u16(d["q"][int(t):int(t) + 1]), kv, want, cfg.sm_scale)
            check_mla(bf16_to_f64(out[i:i + 1]), _np(lse[i:i + 1]), oo, ol, "window row %d" % t)
