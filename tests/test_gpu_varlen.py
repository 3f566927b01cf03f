"""GPU parity of attention over packed variable-length sequences (through the
C ABI) against the fp64 oracle applied to each sequence alone, on seeded
inputs, at the bf16 attention bar (2e-2 on O, 1e-3 on lse).  Packed attention
is, by definition, independent attention per sequence."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


@pytest.fixture(scope="module")
def osm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_08_amd
    return online_softmax_08_amd


def _packed(lengths, H, d, seed):
    # Q, K, V drawn by the attention recipe as one [1, H, total, d] block:
    # sequence b is rows cu[b] .. cu[b+1] - 1 of every head.
    total = int(sum(lengths))
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q, k, v = inputs.attn_inputs(base, B=1, H=H, N=total, d=d, seed=seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q[0], k[0], v[0], cu


def _gpu_varlen(osm, q, k, v, cu, causal):
    dev = torch.device("cuda:0")
    cu_t = torch.from_numpy(cu).to(dev)
    O, lse = osm.attention_varlen(q.to(dev), k.to(dev), v.to(dev), cu_t,
                                  int(np.max(np.diff(cu))) if len(cu) > 1 else 0, causal=causal)
    torch.cuda.synchronize()
    return O.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H", [2, 8])
def test_varlen_against_per_sequence_oracle(osm, H, d, causal):
    # With 2 heads the packed 64-row (4-wave) kernel runs, with 8 heads the
    # 128-row one under the mask and the phase-staggered one without it.
    lengths = [1, 100, 0, 256, 513, 1000, 64, 65]
    q, k, v, cu = _packed(lengths, H=H, d=d, seed=700 + d + H)
    print(f"varlen H={H} d={d} causal={causal} lengths={lengths}", flush=True)
    O, lse = _gpu_varlen(osm, q, k, v, cu, causal)
    eo = el = 0.0
    for b in range(len(lengths)):
        a, e = int(cu[b]), int(cu[b + 1])
        if a == e:
            continue
        Oref, lref = oracle.attn_fwd(q[None, :, a:e], k[None, :, a:e], v[None, :, a:e],
                                     1.0 / math.sqrt(d), causal)
        eo = max(eo, float(np.max(np.abs(O[:, a:e] - Oref[0]))))
        el = max(el, float(np.max(np.abs(lse[:, a:e] - lref[0]))))
    print(f"  max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_attn_fwd(osm, causal):
    # B equal sequences of length L packed: bitwise the dense call on the
    # same rows ([B, H, L, d] <-> [H, B*L, d]).
    B, H, L, d = 4, 16, 1024, 128
    q, k, v, cu = _packed([L] * B, H, d, seed=800)
    dev = torch.device("cuda:0")
    O, lse = osm.attention_varlen(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(cu).to(dev), L,
                                  causal=causal)
    dense = lambda t: t.view(H, B, L, d).permute(1, 0, 2, 3).contiguous().to(dev)
    Od, lsed = osm.attention(dense(q), dense(k), dense(v), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(O.view(H, B, L, d).permute(1, 0, 2, 3), Od)
    assert torch.equal(lse.view(H, B, L).permute(1, 0, 2), lsed)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_long_mixed_full(osm, d, causal):
    # Mixed lengths up to 4096 (the padded layout would waste half its rows),
    # 16 heads: 2048 query blocks of 256 rows, so the packed twin of the
    # phase-staggered kernel runs, at both head sizes and under both masks.
    # Every row of every sequence against the oracle on that sequence alone.
    lengths = [4096, 17, 2048, 3000, 1, 900, 4000, 255]
    H = 16
    q, k, v, cu = _packed(lengths, H, d, seed=900 + d)
    O, lse = _gpu_varlen(osm, q, k, v, cu, causal)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    eo = el = 0.0
    for b, n in enumerate(lengths):
        a = int(cu[b])
        Oref, lref = oracle.attn_fwd(q[None, :, a:a + n], k[None, :, a:a + n], v[None, :, a:a + n],
                                     1.0 / math.sqrt(d), causal)
        eo = max(eo, float(np.max(np.abs(O[:, a:a + n] - Oref[0]))))
        el = max(el, float(np.max(np.abs(lse[:, a:a + n] - lref[0]))))
    print(f"varlen long d={d} causal={causal}: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(2, 2), (4, 2)])
def test_varlen_backward_against_per_sequence_oracle(osm, heads, causal):
    # Gradients of packed sequences (from the packed forward's own O and lse)
    # against the oracle's gradients of each sequence alone; with fewer
    # key/value heads the oracle repeats them and sums the gradient copies.
    H, Hkv = heads
    G = H // Hkv
    lengths = [130, 1, 0, 257, 64, 500]
    d = 64
    total = sum(lengths)
    base = inputs.ATTN["attn_bf16_B2H8N1024d64"]
    q = inputs.attn_inputs(base, B=1, H=H, N=total, d=d, seed=950)[0][0]
    _, k, v = inputs.attn_inputs(base, B=1, H=Hkv, N=total, d=d, seed=951)
    k, v = k[0], v[0]
    g = inputs.grad_output(q.shape, 952)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    cu_t = torch.from_numpy(cu).to(dev)
    O, lse = osm.attention_varlen(qd, kd, vd, cu_t, max(lengths), causal=causal)
    dq, dk, dv = osm.attention_varlen_backward(qd, kd, vd, O, lse, gd, cu_t, max(lengths),
                                               causal=causal)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    errs, scales = [0.0] * 3, [1.0] * 3
    for b in range(len(lengths)):
        a, e = int(cu[b]), int(cu[b + 1])
        if a == e:
            continue
        rq, rk, rv = oracle.attn_bwd(q[None, :, a:e], k[None, :, a:e].repeat_interleave(G, dim=1),
                                     v[None, :, a:e].repeat_interleave(G, dim=1), g[None, :, a:e],
                                     1 / math.sqrt(d), causal)
        rk = rk[0].reshape(Hkv, G, e - a, d).sum(axis=1)
        rv = rv[0].reshape(Hkv, G, e - a, d).sum(axis=1)
        for i, (x, r) in enumerate(zip(got, (rq[0], rk, rv))):
            errs[i] = max(errs[i], float(np.max(np.abs(x[:, a:e] - r))))
            scales[i] = max(scales[i], float(np.max(np.abs(r))))
    print(f"varlen bwd H{H}Hkv{Hkv} causal={causal}: errs={[f'{x:.3e}' for x in errs]} "
          f"bars={[f'{2e-2 * s:.3e}' for s in scales]}", flush=True)
    assert all(np.isfinite(x).all() for x in got)
    assert all(e <= 2e-2 * s for e, s in zip(errs, scales))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,heads", [(128, (4, 4)), (64, (8, 4))])
def test_varlen_backward_eight_wave(osm, d, heads, causal):
    # Long packed sequences (8 of them, up to 4096) with 4 key/value heads:
    # enough 256-row blocks that both backward kernels run their packed
    # 8-wave workgroups (at d = 64 with two query heads per key/value head).
    # Four sequences, of lengths 17, 2048, 3000 and 255, against the oracle's
    # gradients of each sequence alone.
    H, Hkv = heads
    G = H // Hkv
    lengths = [4096, 17, 2048, 3000, 1, 900, 4000, 255]
    total = sum(lengths)
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q = inputs.attn_inputs(base, B=1, H=H, N=total, d=d, seed=960 + d)[0][0]
    _, k, v = inputs.attn_inputs(base, B=1, H=Hkv, N=total, d=d, seed=961 + d)
    k, v = k[0], v[0]
    g = inputs.grad_output(q.shape, 962 + d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    cu_t = torch.from_numpy(cu).to(dev)
    O, lse = osm.attention_varlen(qd, kd, vd, cu_t, max(lengths), causal=causal)
    dq, dk, dv = osm.attention_varlen_backward(qd, kd, vd, O, lse, gd, cu_t, max(lengths),
                                               causal=causal)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    assert all(np.isfinite(x).all() for x in got)
    errs, scales = [0.0] * 3, [1.0] * 3
    for b in (1, 2, 3, 7):
        a, e = int(cu[b]), int(cu[b + 1])
        rq, rk, rv = oracle.attn_bwd(q[None, :, a:e], k[None, :, a:e].repeat_interleave(G, dim=1),
                                     v[None, :, a:e].repeat_interleave(G, dim=1), g[None, :, a:e],
                                     1 / math.sqrt(d), causal)
        rk = rk[0].reshape(Hkv, G, e - a, d).sum(axis=1)
        rv = rv[0].reshape(Hkv, G, e - a, d).sum(axis=1)
        for i, (x, r) in enumerate(zip(got, (rq[0], rk, rv))):
            errs[i] = max(errs[i], float(np.max(np.abs(x[:, a:e] - r))))
            scales[i] = max(scales[i], float(np.max(np.abs(r))))
    print(f"varlen bwd 8-wave d={d} H{H}Hkv{Hkv} causal={causal}: errs={[f'{x:.3e}' for x in errs]} "
          f"bars={[f'{2e-2 * s:.3e}' for s in scales]}", flush=True)
    assert all(e <= 2e-2 * s for e, s in zip(errs, scales))
