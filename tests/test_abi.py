"""The C ABI without a GPU: the library loads, exports every declared entry point, and
rejects invalid arguments before any HIP call (so these run on a CPU-only host)."""
import ctypes
import os
import re

import pytest

import sparse_attention_05_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        from sparse_attention_05_amd import build
        build.build()
    return dsa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(dsa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.dsa_version() == 105
    for code, name in [(0, b"DSA_OK"), (1, b"DSA_ERR_INVALID_ARGUMENT"),
                       (2, b"DSA_ERR_UNSUPPORTED"), (3, b"DSA_ERR_WORKSPACE_TOO_SMALL"),
                       (4, b"DSA_ERR_HIP")]:
        assert lib.dsa_status_string(code) == name


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first


def idx_scores(lib, T=4, L=8, H_I=4, q_pos0=0, c=0.1, ld=8, ptr=FAKE, qp=FAKE):
    return lib.dsa_index_scores(qp, ptr, ptr, ptr, ptr, T, L, H_I, q_pos0, c, ptr, ld, 1, NULL)


def test_index_scores_validation(lib):
    assert idx_scores(lib, ptr=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert idx_scores(lib, T=-1) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert idx_scores(lib, q_pos0=5) == dsa.DSA_ERR_INVALID_ARGUMENT      # q_pos0 + T > L
    assert idx_scores(lib, ld=7) == dsa.DSA_ERR_INVALID_ARGUMENT          # ld < L
    assert idx_scores(lib, c=0.0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert idx_scores(lib, c=float("nan")) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert idx_scores(lib, H_I=3) == dsa.DSA_ERR_UNSUPPORTED
    assert idx_scores(lib, H_I=256) == dsa.DSA_ERR_UNSUPPORTED
    assert idx_scores(lib, qp=ctypes.c_void_p((1 << 20) + 4)) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert idx_scores(lib, T=0, ptr=NULL, qp=NULL) == dsa.DSA_OK           # empty: no launch


def test_topk_validation(lib):
    f = lambda T=4, L=8, q=0, k=2, ld=8, p=FAKE: lib.dsa_topk(p, ld, T, L, q, k, p, NULL, 0, NULL)
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(k=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(k=8193) == dsa.DSA_ERR_UNSUPPORTED
    assert f(ld=4) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(q=6) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(T=0, p=NULL) == dsa.DSA_OK
    assert lib.dsa_topk_workspace_bytes(100, 1000, 10) == 0


def test_sparse_mla_validation(lib):
    f = lambda T=4, L=8, H=16, k=4, s=0.05, p=FAKE: lib.dsa_sparse_mla(p, p, p, T, L, H, k, s, p, p, NULL)
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H=129) == dsa.DSA_ERR_UNSUPPORTED
    assert f(k=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(s=-1.0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(L=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(T=0, p=NULL) == dsa.DSA_OK
    # a cache of more than 2 GiB of 1152-byte rows is beyond the gather's row offsets
    assert f(T=1, L=1864136) == dsa.DSA_ERR_UNSUPPORTED


def test_prefill_validation_and_workspace(lib):
    need = lib.dsa_prefill_workspace_bytes(1024, 1024, 4, 8, 256)
    assert need > 1024 * 1024 * 4
    assert lib.dsa_prefill_workspace_bytes(0, 1024, 4, 8, 256) == 0
    assert lib.dsa_prefill_chunk_rows(131072, 131072) == 4096
    assert lib.dsa_prefill_chunk_rows(2048, 2048) == 2048
    assert lib.dsa_prefill_chunk_rows(0, 10) == 0

    def f(T=16, L=16, H_I=4, H=16, k=4, q=0, ws=FAKE, wsb=None, p=FAKE):
        wsb = need if wsb is None else wsb
        return lib.dsa_prefill(p, p, p, p, p, p, p, T, L, H_I, H, k, q, 0.1, 0.05, p, p, NULL,
                               ws, wsb, NULL)
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(q=1) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H_I=5) == dsa.DSA_ERR_UNSUPPORTED
    assert f(k=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(ws=NULL) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(wsb=1) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(ws=ctypes.c_void_p((1 << 20) + 128)) == dsa.DSA_ERR_INVALID_ARGUMENT  # alignment
    assert f(L=1864136) == dsa.DSA_ERR_UNSUPPORTED                  # cache beyond 2 GiB


def test_decode_validation_and_workspace(lib):
    need = lib.dsa_decode_workspace_bytes(4, 100, 300, 64, 128, 64)
    assert need >= 300 * 4 + 4 * 64 * 4

    def f(B=4, ml=100, N=300, H_I=64, H=128, k=64, ws=FAKE, wsb=None, p=FAKE):
        wsb = need if wsb is None else wsb
        return lib.dsa_decode(B, p, ml, N, p, p, p, p, p, p, p, H_I, H, k, 0.1, 0.05, p, p,
                              NULL, ws, wsb, NULL)
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(N=401) == dsa.DSA_ERR_INVALID_ARGUMENT       # more tokens than B * max_len
    assert f(ml=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H_I=48) == dsa.DSA_ERR_UNSUPPORTED
    assert f(ml=1864136) == dsa.DSA_ERR_UNSUPPORTED                 # a sequence beyond 2 GiB
    assert f(ws=NULL) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(B=0, p=NULL) == dsa.DSA_OK


def test_decode_noalloc_validation_and_scratch_limit(lib):
    """The allocation-free decode validates like dsa_decode, and refuses (before any HIP call)
    a batch whose workspace exceeds the library's fixed per-GPU scratch array."""
    cap = lib.dsa_decode_noalloc_scratch_bytes()
    assert cap == 128 << 20

    def f(B=4, ml=100, N=300, H_I=64, H=128, k=64, p=FAKE):
        return lib.dsa_decode_noalloc(B, p, ml, N, p, p, p, p, p, p, p, H_I, H, k, 0.1, 0.05,
                                      p, p, NULL, NULL)
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(N=401) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H_I=48) == dsa.DSA_ERR_UNSUPPORTED
    assert f(B=0, p=NULL) == dsa.DSA_OK
    # the 64-sequence decode batch at 128K fits; four times as many sequences do not
    big = dict(B=64, ml=131072, N=4_199_844, H_I=64, H=128, k=2048)
    assert lib.dsa_decode_workspace_bytes(64, 131072, 4_199_844, 64, 128, 2048) <= cap
    over = dict(big, B=256, N=4 * 4_199_844)
    assert lib.dsa_decode_workspace_bytes(256, 131072, 4 * 4_199_844, 64, 128, 2048) > cap
    assert f(**over) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL


def test_quantize_and_append_validation(lib):
    q = lib.dsa_quantize_fp8
    assert q(FAKE, 0, -1, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert q(FAKE, 2, 4, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT    # dtype flag
    assert q(NULL, 0, 4, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert q(FAKE, 0, 4, NULL, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert q(ctypes.c_void_p((1 << 20) + 8), 0, 4, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert q(NULL, 0, 0, NULL, NULL, NULL) == dsa.DSA_OK                       # nothing to do
    assert q(FAKE, 1, 1 << 40, FAKE, FAKE, NULL) == dsa.DSA_ERR_UNSUPPORTED
    a = lib.dsa_decode_append
    assert a(-1, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert a(2, FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert a(2, NULL, FAKE, 0, FAKE, FAKE, FAKE, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert a(2, FAKE, FAKE, 0, FAKE, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 4),
             NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert a(70000, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, NULL) == dsa.DSA_ERR_UNSUPPORTED
    assert a(0, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL) == dsa.DSA_OK


def test_index_rule_validation(lib):
    w = lib.dsa_window_indices
    assert w(4, 8, 5, 3, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT       # q_pos0 + T > L
    assert w(4, 8, 0, 0, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT       # window < 1
    assert w(4, 8, 0, 3, NULL, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert w(0, 8, 0, 3, NULL, NULL) == dsa.DSA_OK
    u = lib.dsa_local_selected_indices
    assert u(FAKE, 4, 8, 0, 0, 3, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT  # k < 1
    assert u(NULL, 4, 8, 0, 2, 3, FAKE, NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert u(FAKE, 4, 8, 0, 2, (1 << 30), FAKE, NULL) == dsa.DSA_ERR_UNSUPPORTED
    assert u(NULL, 0, 8, 0, 2, 3, NULL, NULL) == dsa.DSA_OK


def test_prefill_varlen_validation_and_workspace(lib):
    def cu(*v):
        return (ctypes.c_int64 * len(v))(*v)
    cq, ck = cu(0, 16, 16, 40), cu(0, 20, 30, 40)       # T = 16, 0, 24; L = 20, 10, 10
    # sequence 2 has T = 24 > L = 10: malformed
    assert lib.dsa_prefill_varlen_workspace_bytes(3, cq, ck, 4, 8, 4) == 0
    cq, ck = cu(0, 16, 16, 40), cu(0, 20, 30, 3000)
    need = lib.dsa_prefill_varlen_workspace_bytes(3, cq, ck, 4, 8, 4)
    assert need == max(lib.dsa_prefill_workspace_bytes(16, 20, 4, 8, 4),
                       lib.dsa_prefill_workspace_bytes(24, 2970, 4, 8, 4))
    assert lib.dsa_prefill_varlen_workspace_bytes(3, cu(0, 0, 0, 0), ck, 4, 8, 4) == 0

    def f(B=3, q_=cq, k_=ck, H_I=4, H=16, k=4, ws=FAKE, wsb=None, p=FAKE):
        wsb = need if wsb is None else wsb
        return lib.dsa_prefill_varlen(B, q_, k_, p, p, p, p, p, p, p, H_I, H, k, 0.1, 0.05,
                                      p, p, NULL, ws, wsb, NULL)
    assert f(B=0, q_=NULL, k_=NULL, p=NULL) == dsa.DSA_OK                 # empty batch
    assert f(q_=cu(0, 0, 0, 0), k_=ck, p=NULL) == dsa.DSA_OK              # no query rows
    assert f(B=-1) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(q_=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(q_=cu(1, 16, 16, 40)) == dsa.DSA_ERR_INVALID_ARGUMENT        # does not start at 0
    assert f(k_=cu(0, 20, 10, 3000)) == dsa.DSA_ERR_INVALID_ARGUMENT      # decreasing
    assert f(q_=cu(0, 21, 21, 40)) == dsa.DSA_ERR_INVALID_ARGUMENT        # T_0 = 21 > L_0 = 20
    assert f(k=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H_I=3) == dsa.DSA_ERR_UNSUPPORTED
    assert f(ws=NULL) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(ws=ctypes.c_void_p((1 << 20) + 128)) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(p=ctypes.c_void_p((1 << 20) + 8)) == dsa.DSA_ERR_INVALID_ARGUMENT  # alignment


def test_warmup_validation_and_workspace(lib):
    need = lib.dsa_indexer_warmup_workspace_bytes(1000, 1000, 64, 16)
    assert need >= 2 * 1000 * 1000 * 4 + 1000 * 16 * 4
    assert lib.dsa_indexer_warmup_workspace_bytes(0, 1000, 64, 16) == 0

    def f(T=16, L=16, H_I=64, H=16, q=0, c=0.1, sm=0.05, ws=FAKE, wsb=None, p=FAKE, dk=FAKE):
        wsb = need if wsb is None else wsb
        return lib.dsa_indexer_warmup(p, p, p, p, p, p, p, T, L, H_I, H, q, c, sm, p, p, p, dk,
                                      NULL, NULL, ws, wsb, NULL)
    assert f(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(dk=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(q=1) == dsa.DSA_ERR_INVALID_ARGUMENT                 # q_pos0 + T > L
    assert f(c=0.0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(sm=float("nan")) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(H_I=8) == dsa.DSA_ERR_UNSUPPORTED                    # warm-up needs H_I >= 16
    assert f(H=129) == dsa.DSA_ERR_UNSUPPORTED
    assert f(T=1 << 25, L=1 << 25, H_I=64) == dsa.DSA_ERR_UNSUPPORTED  # T * H_I >= 2^31
    assert f(ws=NULL) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(wsb=1) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert f(ws=ctypes.c_void_p((1 << 20) + 128)) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert f(p=ctypes.c_void_p((1 << 20) + 8)) == dsa.DSA_ERR_INVALID_ARGUMENT  # alignment

    lse = lambda T=4, L=8, H=8, q=0, sm=0.1, p=FAKE, out=FAKE: lib.dsa_attention_lse(
        p, p, T, L, H, q, sm, out, NULL)
    assert lse(p=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert lse(out=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert lse(q=5) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert lse(H=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert lse(H=200) == dsa.DSA_ERR_UNSUPPORTED
    assert lse(T=0, p=NULL, out=NULL) == dsa.DSA_OK
    dist = lambda ld=8, out=FAKE: lib.dsa_attention_distribution(FAKE, FAKE, FAKE, 4, 8, 8, 0, 0.1,
                                                                 out, ld, NULL)
    assert dist(ld=7) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert dist(out=NULL) == dsa.DSA_ERR_INVALID_ARGUMENT


def test_size_queries_return_full_size_t(lib):
    """Workspace queries are size_t: sizes past 2^32 come back whole through the binding."""
    import sparse_attention_05_amd as m
    for fn in [n for n in m.EXPORTS if n.endswith("_workspace_bytes")]:
        assert getattr(lib, fn).restype is ctypes.c_size_t, fn
    # 3 sequences of 1M tokens with a chunk of queries each: the largest prefill workspace
    cq = (ctypes.c_int64 * 4)(0, 1 << 20, 2 << 20, 3 << 20)
    ck = (ctypes.c_int64 * 4)(0, 1 << 20, 2 << 20, 3 << 20)
    v = lib.dsa_prefill_varlen_workspace_bytes(3, cq, ck, 64, 128, 2048)
    assert v == lib.dsa_prefill_workspace_bytes(1 << 20, 1 << 20, 64, 128, 2048) > 0
    w = lib.dsa_indexer_warmup_workspace_bytes(1 << 20, 1 << 20, 128, 128)
    assert w > (1 << 32)      # the key-gradient partials alone: 8 x 2^20 x 512 bytes


def test_binding_refuses_host_score_matrices(lib):
    """A host tensor never reaches the library as a device pointer."""
    import torch
    with pytest.raises(TypeError):
        dsa.dsa_topk(torch.zeros((4, 8)), 8, 0, 2)


def test_launch_log_prints_one_line_per_call():
    """DSA_LOG=1: each entry-point call prints its name, sizes and status to stderr (checked
    on calls that validation rejects, so no GPU is needed)."""
    import subprocess
    import sys
    code = ("import ctypes, sparse_attention_05_amd as d; lib = d.load(); "
            "lib.dsa_topk(None, 4, -1, 4, 0, 2, None, None, 0, None); "
            "lib.dsa_decode(4, None, 100, 300, *([None] * 7), 64, 128, 64, 0.1, 0.05, None, None, "
            "None, None, 0, None)")
    env = dict(os.environ, DSA_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[dsa] ")]
    assert lines == ["[dsa] dsa_topk T=-1 L=4 q_pos0=0 k=2 -> DSA_ERR_INVALID_ARGUMENT",
                     "[dsa] dsa_decode B=4 max_len=100 total_tokens=300 H_I=64 H=128 k=64 -> "
                     "DSA_ERR_INVALID_ARGUMENT"], r.stderr
    env["DSA_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT)
    assert "[dsa]" not in r.stderr
