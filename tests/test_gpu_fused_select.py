"""The prefill selection without a score round trip (needs an MI355X).

dsa_prefill, for H_I in {64, 128}, L >= 11776 and 2k <= 5888, selects from candidates: a
strided sample of each row's keys gives a threshold, the indexer keeps only the keys at or
above it, and an exact select over those decides the row; rows the candidates cannot decide
(fewer than k of them, or more than fit) are scored in full and selected exactly.  The
selection is the unique top-k of the row (ties to the lower position), so the fused indices
must equal dsa_topk(dsa_index_scores(...)) bit for bit: checked here on every row of the
long workloads and on inputs built to send rows down each fallback.
"""
import pytest
import torch

from parity import report, to_device
from synth import WORKLOADS, PrefillCfg, make_prefill

pytestmark = pytest.mark.gpu

CHUNK = 4096        # rows of one unfused reference call (bounds its fp32 score matrix)


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _fused_idx(dsa, d, k, q_pos0=0):
    T = d["q8"].shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    dsa.dsa_prefill(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"], k, q_pos0,
                    d["score_scale"], d["sm_scale"], idx_out=idx)
    return idx


def _unfused_equal(dsa, d, k, idx, q_pos0=0):
    """Rows of idx that differ from the two-pass composition (counted, first ones named)."""
    T, L = d["q8"].shape[0], d["k8"].shape[0]
    bad = []
    for r0 in range(0, T, CHUNK):
        r1 = min(T, r0 + CHUNK)
        sc = dsa.dsa_index_scores(d["q8"][r0:r1], d["qs"][r0:r1], d["w"][r0:r1], d["k8"],
                                  d["ks"], q_pos0 + r0, d["score_scale"])
        ref = dsa.dsa_topk(sc, L, q_pos0 + r0, k)
        diff = (ref != idx[r0:r1]).any(dim=1).nonzero().flatten()
        bad += (diff + r0).tolist()
        del sc, ref
    return bad


def _cfg(L, k, H_I, H, seed, q_pos0=0, T=None, planted=0.0):
    return PrefillCfg("fused", L=L, k=k, H_I=H_I, H=H, w_std=H_I ** -0.5, seed=seed,
                      q_pos0=q_pos0, T=T, planted_frac=planted)


@pytest.mark.parametrize("L,k,H_I,H,q_pos0,T,planted", [
    # a whole prefill: rows seeing <= k keys, rows whose every key is a candidate
    # (n <= 5888) and rows selected above a sampled threshold
    (12288, 2048, 64, 16, 0, None, 0.01),
    (12000, 64, 64, 8, 0, None, 0.0),
    # a chunk further in, H_I = 128, ragged sizes
    (20001, 2048, 128, 8, 20001 - 3001, 3001, 0.01),
    (16384, 2944, 64, 8, 5000, 7000, 0.0),
    # k = 1: one candidate suffices; the smallest cache the candidate selection takes
    (11776, 1, 64, 8, 0, None, 0.0),
])
def test_fused_selection_equals_two_pass(dsa, L, k, H_I, H, q_pos0, T, planted):
    cfg = _cfg(L, k, H_I, H, seed=L + k + H_I, q_pos0=q_pos0, T=T, planted=planted)
    d = to_device(make_prefill(cfg))
    idx = _fused_idx(dsa, d, k, q_pos0)
    bad = _unfused_equal(dsa, d, k, idx, q_pos0)
    assert not bad, "%d rows differ from the two-pass selection, first %s" % (len(bad), bad[:8])
    report("fused L=%d k=%d H_I=%d" % (L, k, H_I), rows_compared=int(idx.shape[0]),
           rows_differing=0)


@pytest.mark.parametrize("name", ["prefill-L32768-k2048", "prefill-L131072-k2048"])
def test_fused_selection_every_row_of_the_long_workloads(dsa, name):
    """All 32768 / 131072 rows of the benchmark's workloads, as the benchmark runs them."""
    cfg = WORKLOADS[name]
    d = make_prefill(cfg, device="cuda")
    idx = _fused_idx(dsa, d, cfg.k)
    del d["q"], d["kv"]
    torch.cuda.empty_cache()
    bad = _unfused_equal(dsa, d, cfg.k, idx)
    assert not bad, "%d rows differ from the two-pass selection, first %s" % (len(bad), bad[:8])
    report(name, fused_rows_compared=int(idx.shape[0]), fused_rows_differing=0)


def test_fused_selection_falls_back_when_candidates_cannot_decide(dsa):
    """Two inputs that defeat the candidates.  (1) Every key equal: every score ties, so rows
    longer than the candidate capacity keep all their keys as candidates and overflow; the
    exact path must return positions 0..k-1.  (2) Boosted key scales at every 64th position
    (the sample's stride at this length) with positive weights: the sample sees only the
    boosted keys, the threshold lands above all but a few dozen keys, and the rows have fewer
    than k candidates."""
    L, k, H_I, H = 16384, 2048, 64, 8
    cfg = _cfg(L, k, H_I, H, seed=77)
    d = to_device(make_prefill(cfg))

    same = dict(d)
    same["k8"] = d["k8"][:1].expand(L, 128).contiguous()
    same["ks"] = torch.full_like(d["ks"], float(d["ks"][0]))
    idx = _fused_idx(dsa, same, k)
    bad = _unfused_equal(dsa, same, k, idx)
    assert not bad, "ties: %d rows differ, first %s" % (len(bad), bad[:8])
    first = torch.arange(k, dtype=torch.int32, device="cuda")
    assert torch.equal(idx[k:], first.expand(L - k, k)), "ties go to the lowest positions"

    boosted = dict(d)
    boosted["w"] = d["w"].abs()
    ks = d["ks"].clone()
    ks[::64] *= 64.0
    boosted["ks"] = ks
    idx = _fused_idx(dsa, boosted, k)
    bad = _unfused_equal(dsa, boosted, k, idx)
    assert not bad, "sparse sample: %d rows differ, first %s" % (len(bad), bad[:8])
    report("fused fallbacks", rows_compared=2 * L, rows_differing=0)


@pytest.mark.parametrize("group", [200, 300])
def test_fused_selection_ties_at_the_boundary(dsa, group):
    """Keys tied at the k-th score.  `group` positions, spread over the cache, hold the same
    boosted key (same fp8 row, same scale) and the weights are positive, so for every row that
    sees more than k of them the k-th largest score is the group's and the selection must keep
    the k group positions of lowest index.  With 200 tied candidates the resolve ranks the
    ties itself; with 300 (more than its tie list holds) the row takes the exact path."""
    L, k, H_I, H = 16384, 64, 64, 8
    cfg = _cfg(L, k, H_I, H, seed=91 + group)
    d = to_device(make_prefill(cfg))
    d["w"] = d["w"].abs()
    g = torch.Generator().manual_seed(group)
    pos = torch.randperm(L, generator=g)[:group].sort().values.to("cuda")
    k8 = d["k8"].clone()
    k8[pos] = k8[pos[0]].clone()
    ks = d["ks"].clone()
    ks[pos] = float(ks.max()) * 8.0
    d["k8"], d["ks"] = k8, ks
    idx = _fused_idx(dsa, d, k)
    bad = _unfused_equal(dsa, d, k, idx)
    assert not bad, "ties: %d rows differ, first %s" % (len(bad), bad[:8])
    # the last row sees every group position; whatever tau is, the group positions it keeps
    # are the lowest ones of the group
    sel = set(idx[-1].tolist())
    kept = [p for p in pos.tolist() if p in sel]
    assert kept == pos.tolist()[:len(kept)], "tied positions kept out of order"
    report("fused ties group=%d" % group, rows_compared=L, rows_differing=0,
           last_row_group_kept=len(kept))
