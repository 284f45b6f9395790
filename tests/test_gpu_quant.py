"""fp8 preparation of the indexer inputs and the decode cache append: HIP path vs the CPU
oracle, byte for byte, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _test_vectors(seed):
    """Random vectors over 60 orders of magnitude, every e4m3fn value, midpoint and midpoint
    neighbour at scale 1 (both signs), all-zero, negative-zero and one-hot vectors."""
    g = torch.Generator().manual_seed(seed)
    parts = [torch.randn((40, 128), generator=g) * m for m in (1e-30, 1e-3, 1.0, 7.0, 1e5, 1e30)]
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    mids = (vals[1:] + vals[:-1]) / 2
    pool = torch.cat([vals, mids, torch.nextafter(mids, torch.full_like(mids, 1e9)),
                      torch.nextafter(mids, torch.zeros_like(mids))])
    pool = torch.cat([pool, -pool])
    n = (len(pool) + 126) // 127
    ties = torch.zeros((n, 128))
    ties[:, 1:] = torch.cat([pool, torch.zeros(n * 127 - len(pool))]).view(n, 127)
    ties[:, 0] = 448.0
    special = torch.zeros((3, 128))
    special[1] = -0.0
    special[2, 77] = -3.0
    return torch.cat(parts + [ties, special])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [1, 15, 17, None])
def test_quantize_fp8_matches_oracle(dsa, dtype, n):
    x = _test_vectors(11).to(dtype)
    if n is not None:
        x = x[:n].contiguous()
    q8, sc = dsa.dsa_quantize_fp8(x.cuda())
    torch.cuda.synchronize()
    oq, osc = oracle.quantize_e4m3(_bits(x) if dtype == torch.bfloat16 else x.numpy())
    assert np.array_equal(_np(sc), osc)
    assert np.array_equal(_np(q8), oq)


def test_quantize_fp8_every_fp32_value_of_magnitude_at_most_448(dsa):
    """Each fp32 value with |x| <= 448, both signs, zero and the subnormals included (2.28e9
    values), quantised at scale 1 (every vector also holds 448, its amax, so x / scale = x):
    the codes equal torch's e4m3fn cast (round to nearest even) on the same values.  This pins
    the rounding of a quotient to a code exhaustively; the other tests pin the scale and the
    quotient against the oracle."""
    top = 0x43E00000                                 # 448.0
    batch = 127 << 20                                # values per call (127 per vector)
    for start in range(0, top + 1, batch):
        n = min(batch, top + 1 - start)
        bits = torch.arange(start, start + n, dtype=torch.int32, device="cuda")
        for sign in (0, -(1 << 31)):
            nv = (n + 126) // 127
            flat = torch.zeros(nv * 127, dtype=torch.int32, device="cuda")
            flat[:n] = bits | sign
            x = torch.cat([torch.full((nv, 1), 448.0, device="cuda"),
                           flat.view(torch.float32).view(nv, 127)], dim=1).contiguous()
            q8, sc = dsa.dsa_quantize_fp8(x)
            want = x.to(torch.float8_e4m3fn).view(torch.uint8)
            assert bool((sc == 1.0).all()), "scale of a vector whose amax is 448"
            bad = (q8.view(torch.uint8) != want).nonzero()
            assert bad.numel() == 0, "first mismatch at value bits %#x" % (
                int(x[bad[0, 0], bad[0, 1]].view(torch.int32)) & 0xFFFFFFFF)
            del flat, x, q8, sc, want
        del bits
        torch.cuda.empty_cache()


def test_quantize_fp8_prefill_inputs_sampled(dsa):
    """The indexer inputs of the 128K prefill (131072 x 64 query vectors and 131072 key
    vectors, bf16), quantised in one call; sampled vectors against the oracle."""
    cfg = WORKLOADS["prefill-L131072-k2048"]
    n = cfg.L * cfg.H_I + cfg.L
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((n, 128), generator=g, device="cuda").to(torch.bfloat16)
    q8, sc = dsa.dsa_quantize_fp8(x)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(1).integers(0, n, 3000), [0, n - 1]]))
    ri = torch.from_numpy(rows).cuda()
    oq, osc = oracle.quantize_e4m3(_bits(x[ri]))
    assert np.array_equal(_np(sc[ri]), osc)
    assert np.array_equal(_np(q8[ri]), oq)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_append_matches_oracle(dsa, dtype):
    rng = np.random.default_rng(8)
    lens = np.array([1, 5, 300, 2, 17, 4096, 3])
    st = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, B = int(st[-1]), len(lens)
    k8 = rng.integers(0, 256, (N, 128), dtype=np.uint8)
    ks = rng.random(N).astype(np.float32)
    kv = rng.integers(0, 65536, (N, 576), dtype=np.uint16)
    g = torch.Generator().manual_seed(2)
    k_new = (torch.randn((B, 128), generator=g) * 3).to(dtype)
    kv_new = torch.randn((B, 576), generator=g).to(torch.bfloat16)
    dk8, dks = torch.from_numpy(k8.copy()).cuda(), torch.from_numpy(ks.copy()).cuda()
    dkv = torch.from_numpy(kv.copy().view(np.int16)).view(torch.bfloat16).cuda()
    dsa.dsa_decode_append(torch.from_numpy(st).cuda(), k_new.cuda(), kv_new.cuda(), dk8, dks, dkv)
    torch.cuda.synchronize()
    oracle.decode_append(st, _bits(k_new) if dtype == torch.bfloat16 else k_new.numpy(),
                         _bits(kv_new), k8, ks, kv)
    assert np.array_equal(_np(dk8), k8)
    assert np.array_equal(_np(dks), ks)
    assert np.array_equal(_bits(dkv), kv)
