"""GPU parity of grouped- and multi-query attention (K and V with Hkv heads,
query head h reading key/value head h // (H // Hkv)) through the C ABI.

The oracle is the definition: the same attention with each key/value head
repeated for the query heads that read it (numpy/torch repeat, no
arithmetic); for the backward, the gradient of a repeated tensor is the sum
over its copies.  Bars as for the plain paths: forward bf16 2e-2 on O and
1e-3 on lse; backward 2e-2 * max(1, max|ref|) per gradient tensor.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, TOL_G = 2e-2, 1e-3, 2e-2


@pytest.fixture(scope="module")
def osm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_08_amd
    return online_softmax_08_amd


def _case(B, H, Hkv, N, d, seed):
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q, _, _ = inputs.attn_inputs(base, B=B, H=H, N=N, d=d, seed=seed)
    _, k, v = inputs.attn_inputs(base, B=B, H=Hkv, N=N, d=d, seed=seed + 1)
    return q, k, v


def _rep(t, G):
    return t.repeat_interleave(G, dim=t.dim() - 3)


def _maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 8, 2, 300, 64), (1, 8, 1, 257, 128), (2, 4, 4, 100, 128),
                                   (1, 16, 4, 2048, 128)])
def test_gqa_forward_full(osm, shape, causal):
    # The last shape runs the 128-row workgroups with two key groups.
    B, H, Hkv, N, d = shape
    q, k, v = _case(B, H, Hkv, N, d, seed=40 + N + d)
    dev = torch.device("cuda:0")
    O, lse = osm.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    Oref, lref = oracle.attn_fwd(q, _rep(k, H // Hkv), _rep(v, H // Hkv), 1.0 / math.sqrt(d), causal)
    eo, el = _maxabs(O.float().cpu(), Oref), _maxabs(lse.cpu(), lref)
    print(f"gqa B{B}H{H}Hkv{Hkv}N{N}d{d} causal={causal}: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 16, 4, 3000, 128), (1, 32, 8, 3000, 64)])
def test_gqa_phase_staggered_slices(osm, shape, causal):
    # Grids large enough for the phase-staggered kernel (more than 256 blocks
    # of 256 rows), with groups of 4 query heads per key/value head and a
    # ragged N; whole (b, h) slices at the ends of groups against the oracle
    # on the slice's own key/value head.
    B, H, Hkv, N, d = shape
    G = H // Hkv
    q, k, v = _case(B, H, Hkv, N, d, seed=60 + d)
    dev = torch.device("cuda:0")
    O, lse = osm.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    O, lse = O.float().cpu(), lse.cpu()
    worst = (0.0, 0.0)
    for b, h in ((0, 0), (0, G - 1), (B - 1, G), (B - 1, H - 1)):
        kv = h // G
        Oref, lref = oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, kv:kv + 1], v[b:b + 1, kv:kv + 1],
                                     1.0 / math.sqrt(d), causal)
        worst = (max(worst[0], _maxabs(O[b, h], Oref[0, 0])), max(worst[1], _maxabs(lse[b, h], lref[0, 0])))
    print(f"gqa pp B{B}H{H}Hkv{Hkv}N{N}d{d} causal={causal}: max|dO|={worst[0]:.3e} "
          f"max|dlse|={worst[1]:.3e}", flush=True)
    assert worst[0] <= TOL_O and worst[1] <= TOL_LSE


def test_gqa_with_all_heads_is_attn_fwd(osm):
    q, k, v = _case(2, 16, 16, 1024, 128, seed=61)
    dev = torch.device("cuda:0")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    O1, l1 = torch.empty_like(q), torch.empty((2, 16, 1024), device=dev)
    st = torch.cuda.current_stream().cuda_stream
    osm.attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), O1.data_ptr(), l1.data_ptr(),
                     2, 16, 16, 1024, 128, 1 / math.sqrt(128), True, st)
    O2, l2 = osm.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_splitkv_long_rows(osm, causal):
    # Eight query heads on one key/value head, long rows: the library splits.
    B, H, Hkv, N, d = 1, 8, 1, 4096, 128
    ns, _ = osm.attn_fwd_splitkv_plan(B, H, N, d, causal, 0)
    assert ns > 1
    q, k, v = _case(B, H, Hkv, N, d, seed=71)
    dev = torch.device("cuda:0")
    O, lse = osm.attention_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, 255, 256, 2047, N - 1, *rng.choice(N, size=20, replace=False).tolist()})
    bh = np.array([s for s in range(H) for _ in rows])
    qi = np.array(rows * H)
    Oref, lref = oracle.attn_rows(q, _rep(k, H), _rep(v, H), 1 / math.sqrt(d), causal, bh, qi)
    Og = O.float().cpu().numpy().reshape(H, N, d)[bh, qi]
    lg = lse.cpu().numpy().reshape(H, N)[bh, qi]
    eo, el = _maxabs(Og, Oref), _maxabs(lg, lref)
    print(f"gqa split nsplit={ns} causal={causal}: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


def test_gqa_varlen(osm):
    lengths = [300, 1, 0, 129, 64]
    H, Hkv, d = 4, 2, 64
    total = sum(lengths)
    base = inputs.ATTN["attn_bf16_B2H8N1024d64"]
    q = inputs.attn_inputs(base, B=1, H=H, N=total, d=d, seed=81)[0][0]
    _, k, v = inputs.attn_inputs(base, B=1, H=Hkv, N=total, d=d, seed=82)
    k, v = k[0], v[0]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = torch.device("cuda:0")
    O, lse = osm.attention_varlen(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(cu).to(dev),
                                  max(lengths), causal=True)
    torch.cuda.synchronize()
    O, lse = O.float().cpu().numpy(), lse.cpu().numpy()
    eo = el = 0.0
    for b in range(len(lengths)):
        a, e = int(cu[b]), int(cu[b + 1])
        if a == e:
            continue
        Oref, lref = oracle.attn_fwd(q[None, :, a:e], _rep(k[None, :, a:e], H // Hkv),
                                     _rep(v[None, :, a:e], H // Hkv), 1 / math.sqrt(d), True)
        eo = max(eo, _maxabs(O[:, a:e], Oref[0]))
        el = max(el, _maxabs(lse[:, a:e], lref[0]))
    print(f"gqa varlen: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 256, 64), (1, 8, 1, 200, 128), (1, 8, 2, 1024, 128)])
def test_gqa_backward_full(osm, shape, causal):
    B, H, Hkv, N, d = shape
    G = H // Hkv
    q, k, v = _case(B, H, Hkv, N, d, seed=90 + N + d)
    g = inputs.grad_output(q.shape, 91 + N)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    O, lse = osm.attention(qd, kd, vd, causal=causal)
    dq, dk, dv = osm.attention_backward(qd, kd, vd, O, lse, gd, causal=causal)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    rq, rk, rv = oracle.attn_bwd(q, _rep(k, G), _rep(v, G), g, 1 / math.sqrt(d), causal)
    rk = rk.reshape(B, Hkv, G, N, d).sum(axis=2)
    rv = rv.reshape(B, Hkv, G, N, d).sum(axis=2)
    ok = True
    for name, a, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        e = _maxabs(a.float().cpu(), ref)
        bar = TOL_G * max(1.0, float(np.max(np.abs(ref))))
        print(f"gqa bwd B{B}H{H}Hkv{Hkv}N{N}d{d} causal={causal}: {name} max|err|={e:.3e} bar={bar:.3e}",
              flush=True)
        ok &= e <= bar
    assert ok


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_eight_wave(osm, causal):
    # Grids where both backward kernels run 8-wave workgroups (key blocks x
    # key/value heads and query blocks x query heads each at least 256), with
    # the dK/dV workgroup walking the 2 query heads of its group: the
    # gradients of two whole key/value heads (and their 4 query heads)
    # against the oracle on repeated heads.
    B, H, Hkv, N, d = 2, 32, 16, 2048, 128
    G = H // Hkv
    q, k, v = _case(B, H, Hkv, N, d, seed=95)
    g = inputs.grad_output(q.shape, 96)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    O, lse = osm.attention(qd, kd, vd, causal=causal)
    dq, dk, dv = osm.attention_backward(qd, kd, vd, O, lse, gd, causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = (t.float().cpu() for t in (dq, dk, dv))
    ok = True
    for b, kv in ((0, 0), (B - 1, Hkv - 1)):
        hs = slice(kv * G, kv * G + G)
        rq, rk, rv = oracle.attn_bwd(q[b:b + 1, hs], _rep(k[b:b + 1, kv:kv + 1], G),
                                     _rep(v[b:b + 1, kv:kv + 1], G), g[b:b + 1, hs],
                                     1 / math.sqrt(d), causal)
        for name, a, ref in (("dQ", dq[b:b + 1, hs], rq), ("dK", dk[b, kv], rk.sum(axis=1)[0]),
                             ("dV", dv[b, kv], rv.sum(axis=1)[0])):
            e = _maxabs(a, ref)
            bar = TOL_G * max(1.0, float(np.max(np.abs(ref))))
            print(f"gqa bwd 8-wave b{b} kv{kv} causal={causal}: {name} max|err|={e:.3e} bar={bar:.3e}",
                  flush=True)
            ok &= e <= bar
    assert ok


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_split_auto(osm, causal):
    # attn_bwd_split with the library's count on grouped queries: the count
    # follows the key/value heads ([2, 16/4, 2048, 128]: 64 key blocks, so 4
    # ranges), the dK/dV loop walking a range of its group's query heads and
    # tiles.  The gradients of two whole key/value heads (and their 4 query
    # heads each) against the oracle on repeated heads.
    B, H, Hkv, N, d = 2, 16, 4, 2048, 128
    G = H // Hkv
    assert osm.attn_bwd_split_plan(B, H, Hkv, N, d, causal, 0)[0] == 4
    q, k, v = _case(B, H, Hkv, N, d, seed=97)
    g = inputs.grad_output(q.shape, 98)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    O, lse = osm.attention(qd, kd, vd, causal=causal)
    dq, dk, dv = osm.attention_backward_split(qd, kd, vd, O, lse, gd, causal=causal, nsplit=0)
    torch.cuda.synchronize()
    dq, dk, dv = (t.float().cpu() for t in (dq, dk, dv))
    ok = True
    for b, kv in ((0, 0), (B - 1, Hkv - 1)):
        hs = slice(kv * G, kv * G + G)
        rq, rk, rv = oracle.attn_bwd(q[b:b + 1, hs], _rep(k[b:b + 1, kv:kv + 1], G),
                                     _rep(v[b:b + 1, kv:kv + 1], G), g[b:b + 1, hs],
                                     1 / math.sqrt(d), causal)
        for name, a, ref in (("dQ", dq[b:b + 1, hs], rq), ("dK", dk[b, kv], rk.sum(axis=1)[0]),
                             ("dV", dv[b, kv], rv.sum(axis=1)[0])):
            e = _maxabs(a, ref)
            bar = TOL_G * max(1.0, float(np.max(np.abs(ref))))
            print(f"gqa bwd split auto b{b} kv{kv} causal={causal}: {name} max|err|={e:.3e} bar={bar:.3e}",
                  flush=True)
            ok &= e <= bar
    assert ok
