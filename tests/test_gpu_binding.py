"""The Python binding refuses caller buffers the kernels could not use -- host tensors, score
matrices narrower than L, non-contiguous workspaces -- before anything is launched (needs an
MI355X for the device-side inputs; no kernel runs)."""
import pytest
import torch

from synth import PrefillCfg, make_prefill

pytestmark = pytest.mark.gpu


def _inputs():
    cfg = PrefillCfg("bind", L=64, k=16, H_I=4, H=8, w_std=0.5, seed=3)
    return cfg, make_prefill(cfg, device="cuda")


def test_host_or_narrow_score_matrices_are_refused(dsa):
    cfg, d = _inputs()
    args = (d["q8"], d["qs"], d["w"], d["k8"], d["ks"], 0, cfg.score_scale)
    with pytest.raises(TypeError):
        dsa.dsa_index_scores(*args, scores=torch.empty((64, 64)))
    with pytest.raises(ValueError):
        dsa.dsa_index_scores(*args, scores=torch.empty((64, 63), device="cuda"))
    with pytest.raises(TypeError):
        dsa.dsa_topk(torch.zeros((64, 64)), 64, 0, 16)
    with pytest.raises(ValueError):
        dsa.dsa_topk(torch.zeros((64, 32), device="cuda"), 64, 0, 16)
    lse = torch.zeros((64, 8), device="cuda")
    with pytest.raises(TypeError):
        dsa.dsa_attention_distribution(d["q"], d["kv"], lse, 0, cfg.sm_scale, P=torch.zeros((64, 64)))


def test_host_or_strided_workspaces_are_refused(dsa):
    cfg, d = _inputs()
    args = (d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"], cfg.k, 0,
            cfg.score_scale, cfg.sm_scale)
    with pytest.raises(TypeError):
        dsa.dsa_prefill(*args, workspace=torch.empty((1 << 20,), dtype=torch.uint8))
    with pytest.raises(TypeError):
        dsa.dsa_prefill(*args, workspace=torch.empty((1 << 21,), dtype=torch.uint8,
                                                     device="cuda")[::2])
    # a workspace of another element type counts in bytes
    need = dsa.dsa_prefill_workspace_bytes(64, 64, 4, 8, cfg.k)
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device="cuda")
    out, lse, _ = dsa.dsa_prefill(*args, workspace=ws)
    ref, rlse, _ = dsa.dsa_prefill(*args)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, rlse)
