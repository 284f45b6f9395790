"""Indexer warm-up (KL to the dense attention distribution, and its gradient) on the HIP path
vs the CPU oracle, through the C ABI (needs an MI355X).

Small cases compare every row and every key; the 32K workload runs in the benchmark's launch
configuration (two 16384-row chunks, the key gradient accumulated across them) and compares
sampled rows, plus the key gradient through the degree-one homogeneity identity
<dk, KI> = sum_{t,h} dw w, which holds at any size (checked to 1e-4 of the sum of the
absolute terms: the bf16 roundings inside dk are independent and cancel in the sum).
Tolerances: tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import WU_LSE_ATOL, WU_P_RTOL, check_warmup_dk, check_warmup_rows
from synth import WORKLOADS, PrefillCfg, make_prefill

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


def _case(L, T, q_pos0, H_I, H, seed):
    cfg = PrefillCfg("warmup", L=L, k=64, H_I=H_I, H=H, w_std=H_I ** -0.5, seed=seed,
                     q_pos0=q_pos0, T=T)
    return make_prefill(cfg, device="cuda")


def _oracle_inputs(d, rows=None):
    """Oracle inputs for the given rows, copying only those rows' queries off the device."""
    T = d["T"]
    r = np.arange(T) if rows is None else np.asarray(rows)
    sel = torch.from_numpy(r).cuda()
    sub = dict(q8=_np(d["q8"][sel]), qs=_np(d["qs"][sel]), w=_np(d["w"][sel]),
               q=_u16(d["q"][sel]), k8=_np(d["k8"]), ks=_np(d["ks"]), kv=_u16(d["kv"]),
               q_pos0=d["q_pos0"], score_scale=d["score_scale"], sm_scale=d["sm_scale"])
    x = oracle.warmup_inputs(sub)
    x["pos"] = d["q_pos0"] + r
    return x


def _run(dsa, d):
    res = dsa.dsa_indexer_warmup(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                                 d["q_pos0"], d["score_scale"], d["sm_scale"])
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in res.items()}


@pytest.mark.parametrize("L,T,q_pos0,H", [(300, 300, 0, 16), (300, 201, 99, 128), (67, 67, 0, 5),
                                          (129, 1, 128, 32)])
def test_attention_lse_and_distribution(dsa, L, T, q_pos0, H):
    d = _case(L, T, q_pos0, 16, H, seed=L + H)
    lse = dsa.dsa_attention_lse(d["q"], d["kv"], q_pos0, d["sm_scale"])
    P = torch.full((T, L + 3), -1.0, dtype=torch.float32, device="cuda")
    dsa.dsa_attention_distribution(d["q"], d["kv"], lse, q_pos0, d["sm_scale"], P=P)
    torch.cuda.synchronize()
    o = oracle.warmup(_oracle_inputs(d), dist=True)
    assert np.abs(_np(lse) - o["lse_t"]).max() <= WU_LSE_ATOL
    g = _np(P)
    vis = np.arange(L + 3)[None, :] <= (q_pos0 + np.arange(T))[:, None]
    assert (g[~vis] == -1.0).all(), "entries past a row's position were written"
    err = np.abs(g[:, :L] - o["P"])[vis[:, :L]]
    tol = (WU_P_RTOL * o["P"] + 1e-9)[vis[:, :L]]
    assert (err <= tol).all(), "P off by %.3g" % (err / np.maximum(tol, 1e-30)).max()


@pytest.mark.parametrize("L,T,q_pos0,H_I,H,seed", [
    (300, 300, 0, 64, 16, 1),       # ragged tiles, odd token count per key tile
    (500, 200, 300, 16, 8, 2),      # a chunk against a cache of 300 tokens, 16 tokens per block
    (257, 257, 0, 128, 32, 3),      # half-token row tiles
    (129, 65, 64, 32, 4, 4),
    (1100, 1100, 0, 64, 16, 5),     # many key tiles and five key blocks
    (400, 100, 50, 64, 8, 7),       # keys 150..399 seen by no row: zero gradient
])
def test_warmup_every_row_and_key(dsa, L, T, q_pos0, H_I, H, seed):
    d = _case(L, T, q_pos0, H_I, H, seed)
    g = _run(dsa, d)
    o = oracle.warmup(_oracle_inputs(d), want_dk=True, bounds=True)
    what = "warmup L=%d T=%d q_pos0=%d H_I=%d H=%d" % (L, T, q_pos0, H_I, H)
    worst = check_warmup_rows(g, o, np.arange(T), what)
    worst["dk"] = check_warmup_dk(g["dk"], o, what)
    print(what, "worst error / tolerance:", {k: round(float(v), 4) for k, v in worst.items()})


def test_warmup_without_query_rows_zeroes_the_key_gradient(dsa):
    d = _case(300, 300, 0, 64, 8, seed=8)
    dk = torch.full((300, 128), 7.0, dtype=torch.float32, device="cuda")
    res = dsa.dsa_indexer_warmup(d["q8"][:0], d["qs"][:0], d["w"][:0], d["k8"], d["ks"],
                                 d["q"][:0], d["kv"], 0, d["score_scale"], d["sm_scale"],
                                 out=dict(dk=dk))
    torch.cuda.synchronize()
    assert res["kl"].shape == (0,) and res["dq"].shape == (0, 64, 128)
    assert (dk == 0).all()


def test_warmup_bitwise_repeatable(dsa):
    d = _case(700, 700, 0, 64, 16, seed=6)
    a, b = _run(dsa, d), _run(dsa, d)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_warmup_32k_sampled_rows_and_key_identity(dsa):
    cfg = WORKLOADS["prefill-L32768-k2048"]
    d = make_prefill(cfg, device="cuda")
    g = _run(dsa, d)
    L = cfg.L
    rows = np.array([0, 1, 63, 64, 2047, 2048, 4095, 4096, 16383, 16384, 16385, 20000, 27313,
                     L - 2, L - 1])
    o = oracle.warmup(_oracle_inputs(d, rows), bounds=True)
    worst = check_warmup_rows(g, o, rows, "warmup 32K")
    print("warmup 32K worst error / tolerance:", {k: round(float(v), 4) for k, v in worst.items()})
    # <dk, KI> = sum_{t,h} dw w = sum_{t,s} G I (both sides from the GPU; dw sampled above)
    KI = oracle.e4m3fn_values(np.arange(256))[_np(d["k8"])] * _np(d["ks"]).astype(np.float64)[:, None]
    lhs_terms = g["dk"].astype(np.float64) * KI
    rhs_terms = g["dw"].astype(np.float64) * _np(d["w"]).astype(np.float64)
    lhs, rhs = lhs_terms.sum(), rhs_terms.sum()
    scale = np.abs(lhs_terms).sum() + np.abs(rhs_terms).sum()
    assert abs(lhs - rhs) <= 1e-4 * scale, (lhs, rhs, scale)
    print("key identity: <dk, KI> = %.6g, sum dw w = %.6g, |diff| / scale = %.3g"
          % (lhs, rhs, abs(lhs - rhs) / scale))
    # keys no row sees do not exist here (T = L); every key has a finite gradient
    assert np.isfinite(g["dk"]).all() and np.isfinite(g["dq"]).all()
