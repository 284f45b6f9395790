"""Seeded synthetic workloads for the DSA hot path.

Every tensor is drawn from one ``torch.Generator`` seeded per workload, in a fixed order,
so a (workload, seed, device) triple always yields the same bytes.  CPU and GPU engines
produce different streams; each side of a comparison is always handed the *same* bytes,
wherever they were drawn.

Storage formats (the contract of the hot path):

* indexer queries ``q8[T, H_I, 128]`` and keys ``k8[L, 128]`` are OCP e4m3fn bytes, each
  128-vector with its own fp32 scale (``qs[T, H_I]``, ``ks[L]``): ``scale = amax / 448``
  (1 when the vector is all zero), code = round-to-nearest-even of ``clamp(v / scale, ±448)``.
  Torch's cast does not saturate (500 -> NaN), hence the clamp.
* MLA queries ``q[T, H, 576]`` and the latent cache ``kv[L, 576]`` (512 latent + 64 rope)
  are bf16, rounded to nearest even from fp32 N(0, 1) draws.
* per-head weights ``w[T, H_I]`` are fp32 N(0, w_std^2).

Planted tokens (the long prefill workloads): a fraction of key positions s get an indexer
key aligned with one query head of a later target row t_s, with the norm of a typical key
(sqrt(128)); only the indexer key changes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

D_I = 128      # indexer key / query width (one shared key per token)
D_QK = 576     # MLA contraction width: 512 latent + 64 rope
D_V = 512      # MLA value width (the latent part of the same cache row)
E4M3_MAX = 448.0


@dataclass(frozen=True)
class PrefillCfg:
    name: str
    L: int                 # keys (cache length)
    k: int                 # selected tokens per query row
    H_I: int               # indexer heads
    H: int                 # MLA heads
    w_std: float           # std of the per-head weights a_h
    seed: int
    planted_frac: float = 0.0
    T: Optional[int] = None    # query rows; default: all L tokens
    q_pos0: int = 0            # absolute position of query row 0
    score_scale: float = D_I ** -0.5
    sm_scale: float = D_QK ** -0.5

    @property
    def rows(self) -> int:
        return self.L - self.q_pos0 if self.T is None else self.T

    def with_(self, **kw) -> "PrefillCfg":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeCfg:
    name: str
    B: int                 # sequences, one query token each
    len_lo: int            # context lengths uniform in [len_lo, len_hi] (inclusive,
    len_hi: int            #   counting the token being decoded)
    k: int
    H_I: int
    H: int
    w_std: float
    seed: int
    score_scale: float = D_I ** -0.5
    sm_scale: float = D_QK ** -0.5

    def with_(self, **kw) -> "DecodeCfg":
        return replace(self, **kw)


@dataclass(frozen=True)
class VarlenCfg:
    """A packed batch of B sequences.  Sequence b holds L_b tokens (uniform in
    [len_lo, len_hi]); its query rows are its last T_b tokens.  Even-numbered sequences are
    fresh prefills (T_b = L_b); odd-numbered ones prefill a chunk of T_b tokens (uniform in
    [chunk_lo, min(chunk_hi, L_b)]) against the cache of their first L_b - T_b tokens."""
    name: str
    B: int
    len_lo: int
    len_hi: int
    chunk_lo: int
    chunk_hi: int
    k: int
    H_I: int
    H: int
    w_std: float
    seed: int
    planted_frac: float = 0.0
    score_scale: float = D_I ** -0.5
    sm_scale: float = D_QK ** -0.5

    def lengths(self):
        """(T_b, L_b) lists drawn from a CPU generator (host-side sizes)."""
        g = torch.Generator()
        g.manual_seed(self.seed)
        L = torch.randint(self.len_lo, self.len_hi + 1, (self.B,), generator=g).tolist()
        u = torch.rand((self.B,), generator=g, dtype=torch.float64).tolist()
        T = []
        for b in range(self.B):
            if b % 2 == 0:
                T.append(L[b])
            else:
                hi = min(self.chunk_hi, L[b])
                lo = min(self.chunk_lo, hi)
                T.append(lo + min(hi - lo, int(u[b] * (hi - lo + 1))))
        return T, L


WORKLOADS = {
    # small prefill, few heads: the case the oracle finishes in seconds
    "prefill-L1024-k256": PrefillCfg("prefill-L1024-k256", L=1024, k=256, H_I=4, H=8,
                                     w_std=0.5, seed=1001),
    # every row sees <= k tokens: must equal dense causal attention
    "prefill-L2048-k2048-dense": PrefillCfg("prefill-L2048-k2048-dense", L=2048, k=2048,
                                            H_I=64, H=128, w_std=1 / 8, seed=1002),
    "prefill-L32768-k2048": PrefillCfg("prefill-L32768-k2048", L=32768, k=2048, H_I=64,
                                       H=128, w_std=1 / 8, seed=1003, planted_frac=0.01),
    "prefill-L131072-k2048": PrefillCfg("prefill-L131072-k2048", L=131072, k=2048, H_I=64,
                                        H=128, w_std=1 / 8, seed=1004, planted_frac=0.01),
    "decode-B64-L4096-131072-k2048": DecodeCfg("decode-B64-L4096-131072-k2048", B=64,
                                               len_lo=4096, len_hi=131072, k=2048, H_I=64,
                                               H=128, w_std=1 / 8, seed=1005),
    # a packed serving batch: 16 sequences of 1K..32K tokens, every other one a chunk of
    # 512..8192 new tokens against its cached prefix (shapes and value distributions of the
    # 32K prefill workload)
    "varlen-B16-L1024-32768-k2048": VarlenCfg("varlen-B16-L1024-32768-k2048", B=16,
                                              len_lo=1024, len_hi=32768, chunk_lo=512,
                                              chunk_hi=8192, k=2048, H_I=64, H=128,
                                              w_std=1 / 8, seed=1006, planted_frac=0.01),
    # many short prompts, each within k (every row selects all it sees): 128 fresh 1K-token
    # prefills
    "varlen-B128-L1024-k2048": VarlenCfg("varlen-B128-L1024-k2048", B=128, len_lo=1024,
                                         len_hi=1024, chunk_lo=1024, chunk_hi=1024, k=2048,
                                         H_I=64, H=128, w_std=1 / 8, seed=1007),
}


def quantize_e4m3_rows(v: torch.Tensor):
    """fp32 [..., n] -> (e4m3fn bytes uint8 [..., n], fp32 scale [...]) per last-dim vector."""
    amax = v.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    code = (v / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return code.view(torch.uint8), scale


def _randn_bf16(g: torch.Generator, shape, device, chunk_rows: int) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to bf16, drawn in row chunks to bound the fp32 temporary."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n = shape[0]
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out


def _chunk_rows(row_elems: int) -> int:
    return max(1, (256 << 20) // (4 * row_elems))   # ~256 MiB of fp32 per draw


def make_prefill(cfg: PrefillCfg, device="cpu", seed: Optional[int] = None) -> dict:
    """Inputs of one prefill call: T query rows at positions q_pos0.., L cached tokens."""
    device = torch.device(device)
    T, L, H_I, H = cfg.rows, cfg.L, cfg.H_I, cfg.H
    assert 0 <= cfg.q_pos0 and cfg.q_pos0 + T <= L
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed if seed is None else seed)

    q_f = torch.randn((T, H_I, D_I), generator=g, device=device, dtype=torch.float32)
    k_f = torch.randn((L, D_I), generator=g, device=device, dtype=torch.float32)
    w = torch.randn((T, H_I), generator=g, device=device, dtype=torch.float32) * cfg.w_std

    planted = torch.zeros((0, 3), dtype=torch.int64, device=device)
    n_p = int(round(cfg.planted_frac * L))
    if n_p > 0:
        pos = torch.randperm(L, generator=g, device=device)[:n_p]
        u = torch.rand((n_p,), generator=g, device=device, dtype=torch.float64)
        lo = torch.clamp(pos, min=max(cfg.k, cfg.q_pos0))
        keep = lo < cfg.q_pos0 + T
        pos, u, lo = pos[keep], u[keep], lo[keep]
        tgt = lo + torch.floor(u * (cfg.q_pos0 + T - lo).to(torch.float64)).to(torch.int64)
        tgt = torch.minimum(tgt, torch.full_like(tgt, cfg.q_pos0 + T - 1))
        row = tgt - cfg.q_pos0
        head = torch.argmax(w[row], dim=1)
        qv = q_f[row, head]                                   # [n_p, 128]
        k_f[pos] = math.sqrt(D_I) * qv / qv.norm(dim=1, keepdim=True)
        planted = torch.stack([pos, tgt, head], dim=1)

    q8, qs = quantize_e4m3_rows(q_f)
    del q_f
    k8, ks = quantize_e4m3_rows(k_f)
    del k_f
    q = _randn_bf16(g, (T, H, D_QK), device, _chunk_rows(H * D_QK))
    kv = _randn_bf16(g, (L, D_QK), device, _chunk_rows(D_QK))
    return dict(kind="prefill", cfg=cfg, T=T, L=L, H_I=H_I, H=H, k=cfg.k, q_pos0=cfg.q_pos0,
                score_scale=cfg.score_scale, sm_scale=cfg.sm_scale,
                q8=q8.contiguous(), qs=qs.contiguous(), w=w.contiguous(),
                k8=k8.contiguous(), ks=ks.contiguous(), q=q, kv=kv, planted=planted)


def make_varlen(lens_q, lens_k, k: int, H_I: int, H: int, w_std: float, seed: int,
                planted_frac: float = 0.0, device="cpu", name="varlen") -> dict:
    """Packed inputs of B sequences: sequence b contributes T_b = lens_q[b] query rows (its
    last T_b tokens, at positions L_b - T_b ..) and L_b = lens_k[b] cached tokens.  Queries
    are packed along rows by cu_seqlens_q, keys by cu_seqlens_k (host int64 [B + 1]).  Each
    sequence is drawn as its own prefill workload with seed (seed, b)."""
    device = torch.device(device)
    B = len(lens_k)
    assert len(lens_q) == B and all(0 <= t <= l for t, l in zip(lens_q, lens_k))
    cu_q = torch.zeros(B + 1, dtype=torch.int64)
    cu_k = torch.zeros(B + 1, dtype=torch.int64)
    cu_q[1:] = torch.cumsum(torch.tensor(lens_q, dtype=torch.int64), 0)
    cu_k[1:] = torch.cumsum(torch.tensor(lens_k, dtype=torch.int64), 0)
    Tq, Lk = int(cu_q[-1]), int(cu_k[-1])
    out = dict(q8=torch.empty((Tq, H_I, D_I), dtype=torch.uint8, device=device),
               qs=torch.empty((Tq, H_I), dtype=torch.float32, device=device),
               w=torch.empty((Tq, H_I), dtype=torch.float32, device=device),
               q=torch.empty((Tq, H, D_QK), dtype=torch.bfloat16, device=device),
               k8=torch.empty((Lk, D_I), dtype=torch.uint8, device=device),
               ks=torch.empty((Lk,), dtype=torch.float32, device=device),
               kv=torch.empty((Lk, D_QK), dtype=torch.bfloat16, device=device))
    for b in range(B):
        if lens_k[b] == 0:
            continue
        cfg = PrefillCfg("%s-seq%d" % (name, b), L=lens_k[b], k=k, H_I=H_I, H=H, w_std=w_std,
                         seed=seed * 1009 + b, planted_frac=planted_frac, T=lens_q[b],
                         q_pos0=lens_k[b] - lens_q[b])
        one = make_prefill(cfg, device)
        qa, qe, ka, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        for key in ("q8", "qs", "w", "q"):
            out[key][qa:qe] = one[key]
        for key in ("k8", "ks", "kv"):
            out[key][ka:ke] = one[key]
        del one
    return dict(kind="varlen", B=B, Tq=Tq, Lk=Lk, H_I=H_I, H=H, k=k,
                lens_q=list(lens_q), lens_k=list(lens_k), cu_q=cu_q, cu_k=cu_k,
                score_scale=D_I ** -0.5, sm_scale=D_QK ** -0.5, **out)


def make_varlen_cfg(cfg: VarlenCfg, device="cpu") -> dict:
    T, L = cfg.lengths()
    d = make_varlen(T, L, cfg.k, cfg.H_I, cfg.H, cfg.w_std, cfg.seed, cfg.planted_frac,
                    device, cfg.name)
    d.update(cfg=cfg, score_scale=cfg.score_scale, sm_scale=cfg.sm_scale)
    return d


def make_decode(cfg: DecodeCfg, device="cpu", seed: Optional[int] = None) -> dict:
    """Inputs of one decode step: B packed ragged caches, one query per sequence at L_b - 1."""
    device = torch.device(device)
    B, H_I, H = cfg.B, cfg.H_I, cfg.H
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed if seed is None else seed)

    lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (B,), generator=g, device=device,
                         dtype=torch.int64)
    seq_start = torch.zeros(B + 1, dtype=torch.int64, device=device)
    seq_start[1:] = torch.cumsum(lens, 0)
    N = int(seq_start[-1].item())

    q_f = torch.randn((B, H_I, D_I), generator=g, device=device, dtype=torch.float32)
    w = torch.randn((B, H_I), generator=g, device=device, dtype=torch.float32) * cfg.w_std
    q8, qs = quantize_e4m3_rows(q_f)
    k8 = torch.empty((N, D_I), dtype=torch.uint8, device=device)
    ks = torch.empty((N,), dtype=torch.float32, device=device)
    step = _chunk_rows(D_I)
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        kf = torch.randn((r1 - r0, D_I), generator=g, device=device, dtype=torch.float32)
        k8[r0:r1], ks[r0:r1] = quantize_e4m3_rows(kf)
    q = _randn_bf16(g, (B, H, D_QK), device, _chunk_rows(H * D_QK))
    kv = _randn_bf16(g, (N, D_QK), device, _chunk_rows(D_QK))
    return dict(kind="decode", cfg=cfg, B=B, N=N, H_I=H_I, H=H, k=cfg.k,
                max_len=int(lens.max().item()), lens=lens, seq_start=seq_start,
                score_scale=cfg.score_scale, sm_scale=cfg.sm_scale,
                q8=q8.contiguous(), qs=qs.contiguous(), w=w.contiguous(), k8=k8, ks=ks,
                q=q, kv=kv)


def host_arrays(inp: dict) -> dict:
    """numpy views of the raw bytes (uint8 fp8 codes, uint16 bf16 bits, fp32, int64)."""
    out = {}
    for key, v in inp.items():
        if isinstance(v, torch.Tensor):
            t = v.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                out[key] = t.view(torch.int16).numpy().view("uint16")
            else:
                out[key] = t.numpy()
        else:
            out[key] = v
    return out
