"""The allocation-free decode entry point against dsa_decode (needs an MI355X).

dsa_decode_noalloc runs the decode kernels on the library's fixed per-GPU scratch array
instead of a caller workspace.  Two calls in a row, the second with a smaller batch (the
array keeps the first call's contents), each compared with dsa_decode on the same inputs:
indices exactly, outputs and lse to the attention rule of tests/parity.py."""
import numpy as np
import pytest
import torch

from parity import check_mla, to_device
from synth import DecodeCfg, make_decode

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _both(dsa, inp):
    d = to_device(inp)
    B, H, k = inp["B"], inp["H"], inp["k"]
    args = (d["seq_start"], inp["max_len"], d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"],
            d["kv"], k, inp["score_scale"], inp["sm_scale"])
    ref_idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ref_out, ref_lse, _ = dsa.dsa_decode(*args, idx_out=ref_idx)
    # caller-owned outputs, filled with garbage first: the call allocates nothing
    out = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device="cuda")
    idx = torch.full((B, k), 7, dtype=torch.int32, device="cuda")
    dsa.dsa_decode_noalloc(*args, out=out, lse=lse, idx_out=idx)
    torch.cuda.synchronize()
    return (ref_out, ref_lse, ref_idx), (out, lse, idx)


@pytest.mark.parametrize("first,second", [
    (dict(B=6, len_lo=1, len_hi=40000, k=2048, H_I=64, H=128),
     dict(B=3, len_lo=1, len_hi=3000, k=256, H_I=64, H=128)),
    (dict(B=4, len_lo=9000, len_hi=20000, k=1024, H_I=4, H=16),
     dict(B=2, len_lo=1, len_hi=500, k=64, H_I=4, H=16)),
])
def test_noalloc_decode_matches_dsa_decode_on_two_calls(dsa, first, second):
    for n, shape in enumerate((first, second)):
        cfg = DecodeCfg("noalloc-%d" % n, w_std=shape["H_I"] ** -0.5, seed=900 + n, **shape)
        inp = make_decode(cfg)
        (ro, rl, ri), (go, gl, gi) = _both(dsa, inp)
        assert np.array_equal(_np(gi), _np(ri)), "call %d: indices differ" % n
        check_mla(_np(go.float()).astype(np.float64), _np(gl), _np(ro.float()).astype(np.float64),
                  _np(rl), "noalloc call %d" % n)


def test_noalloc_decode_refuses_a_batch_beyond_its_scratch(dsa):
    cap = dsa.dsa_decode_noalloc_scratch_bytes()
    B, max_len, N = 256, 131072, 256 * 100000
    assert dsa.dsa_decode_workspace_bytes(B, max_len, N, 64, 128, 2048) > cap
    lib = dsa.load()
    status = lib.dsa_decode_noalloc(B, 1 << 20, max_len, N, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                    1 << 20, 1 << 20, 1 << 20, 64, 128, 2048, 0.1, 0.05,
                                    1 << 20, 1 << 20, None, None)
    assert status == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
