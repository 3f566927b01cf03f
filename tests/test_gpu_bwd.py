"""GPU parity of the attention backward (dQ, dK, dV through the C ABI)
against the fp64 oracle's chain-rule gradients, on seeded inputs.

The GPU backward takes the forward's own bf16 O and fp32 lse as inputs, as a
training step would; the oracle recomputes everything from Q, K, V and dO in
fp64.  Two bars, both enforced:
  * per gradient tensor, max-abs error <= 2e-2 * max(1, max |ref|);
  * per element, |err| <= 6 sigma + u |grad| + 1e-5, with sigma the error
    scale of that element under the bf16 error model of the backward
    (_grad_bounds): the rounding of P before dV, D_i = sum_t dO_it O_it
    formed from the forward's rounded O, the rounding of dS before dK and
    dQ, each rounding at most u = 2^-8 relative, independent and of mean
    zero.  The largest measured ratio of error to this bar is 0.47; a
    regression that corrupts some elements (a missed tile, a wrong mask or
    statistic) exceeds it there even when the tensor's largest error does
    not move.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2  # times max(1, max |ref|) per gradient tensor


@pytest.fixture(scope="module")
def osm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_08_amd
    return online_softmax_08_amd


def _case(B, H, N, d, seed):
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q, k, v = inputs.attn_inputs(base, B=B, H=H, N=N, d=d, seed=seed)
    g = inputs.grad_output(q.shape, seed + 1)
    return q, k, v, g


def _gpu_bwd(osm, q, k, v, g, causal):
    dev = torch.device("cuda:0")
    q, k, v, g = (t.to(dev) for t in (q, k, v, g))
    O, lse = osm.attention(q, k, v, causal=causal)
    dq, dk, dv = osm.attention_backward(q, k, v, O, lse, g, causal=causal)
    torch.cuda.synchronize()
    return [t.to(torch.float64).cpu().numpy() for t in (dq, dk, dv)]


U = 2.0 ** -8       # unit roundoff of bf16 (round to nearest even)
ELEM_FACTOR = 6.0   # per-element bar: ELEM_FACTOR * sigma + u |grad| + ELEM_FLOOR
ELEM_FLOOR = 1e-5


def _grad_bounds(q, k, v, g, scale, causal):
    """Per-element error scale of the bf16 backward, from the error model of
    its rounding steps.  Each rounding of a value x to bf16 errs by at most
    u |x| (u = 2^-8), and the roundings are independent and of mean zero, so
    the error of a sum of such terms has a standard deviation of at most
    u sqrt(sum x^2).  The steps:
      * P rounded before dV = P^T dO: u sqrt(sum_i (P_ij dO_it)^2);
      * D_i = sum_t dO_it O_it from the forward's bf16 O, whose error is at
        most 2u sum_j P_ij |V_jt| (the forward's P rounded, then O rounded):
        dD_i = 2u sqrt(sum_t (dO_it sum_j P_ij |V_jt|)^2), reaching dS_ij as
        P_ij dD_i;
      * dS rounded before dK = scale dS^T Q and dQ = scale dS K: u |dS_ij|;
      * each gradient rounded to bf16 (u |grad|, kept separately).
    Returns (sigma, rounding) pairs for dQ, dK, dV.  The magnitudes are
    evaluated in float64 from the same inputs; they set tolerances only,
    the reference values come from the oracle."""
    Q, Kt, Vt, G = (np.asarray(t.to(torch.float64).numpy()) for t in (q, k, v, g))
    B, H, N, d = Q.shape
    sq, sk, sv = np.zeros_like(Q), np.zeros_like(Q), np.zeros_like(Q)
    rq, rk, rv = np.zeros_like(Q), np.zeros_like(Q), np.zeros_like(Q)
    mask = np.triu(np.ones((N, N), dtype=bool), 1) if causal else None
    for b in range(B):
        for h in range(H):
            qs, ks, vs, gs = Q[b, h], Kt[b, h], Vt[b, h], G[b, h]
            S = scale * (qs @ ks.T)
            if causal:
                S[mask] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O = P @ vs
            D = np.sum(gs * O, axis=1)
            dS = P * (gs @ vs.T - D[:, None])
            dD = 2 * U * np.sqrt(np.sum((gs * (P @ np.abs(vs))) ** 2, axis=1))
            E2 = (P * dD[:, None]) ** 2 + (U * dS) ** 2   # variance scale of dS
            sv[b, h] = U * np.sqrt((P ** 2).T @ gs ** 2)
            sk[b, h] = scale * np.sqrt(E2.T @ qs ** 2)
            sq[b, h] = scale * np.sqrt(E2 @ ks ** 2)
            rv[b, h] = U * np.abs(P.T @ gs)
            rk[b, h] = U * np.abs(scale * (dS.T @ qs))
            rq[b, h] = U * np.abs(scale * (dS @ ks))
    return (sq, rq), (sk, rk), (sv, rv)


def _compare(got, ref, label, bounds=None):
    """Max-abs error within the per-tensor bar and, with bounds, every
    element within ELEM_FACTOR times its error scale plus its own rounding
    (and a small floor)."""
    ok = True
    for x, (name, a, b) in enumerate(zip(("dQ", "dK", "dV"), got, ref)):
        assert np.all(np.isfinite(a)), f"{label}: {name} not finite"
        e = float(np.max(np.abs(a - b))) if a.size else 0.0
        scale = max(1.0, float(np.max(np.abs(b))) if b.size else 0.0)
        msg = f"{label}: {name} max|err|={e:.3e} max|ref|={scale:.3f} bar={TOL * scale:.3e}"
        ok &= e <= TOL * scale
        if bounds is not None and a.size:
            sig, rnd = bounds[x]
            r = np.abs(a - b) / (ELEM_FACTOR * sig + rnd + ELEM_FLOOR)
            msg += f" max err/elem-bar={float(np.max(r)):.3f}"
            ok &= bool(np.all(r <= 1.0))
        print(msg, flush=True)
    assert ok, label


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (1, 2, 256, 128), (2, 1, 200, 128),
                                   (1, 1, 65, 64), (1, 3, 1, 128), (1, 1, 777, 128),
                                   (1, 1, 130, 64)])
def test_bwd_full(osm, shape, causal):
    B, H, N, d = shape
    q, k, v, g = _case(B, H, N, d, seed=5000 + N + d)
    label = f"bwd B{B}H{H}N{N}d{d} causal={causal}"
    print(label, flush=True)
    got = _gpu_bwd(osm, q, k, v, g, causal)
    ref = oracle.attn_bwd(q, k, v, g, 1.0 / math.sqrt(d), causal)
    _compare(got, ref, label, _grad_bounds(q, k, v, g, 1.0 / math.sqrt(d), causal))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_workload(osm, causal):
    # The [2, 8, 1024, 64] workload, every slice.
    w = inputs.ATTN["attn_bf16_B2H8N1024d64"]
    q, k, v = inputs.attn_inputs(w)
    g = inputs.grad_output(q.shape, w.seed + 1)
    label = f"bwd {w.name} causal={causal}"
    print(label, flush=True)
    got = _gpu_bwd(osm, q, k, v, g, causal)
    ref = oracle.attn_bwd(q, k, v, g, w.scale, causal)
    _compare(got, ref, label, _grad_bounds(q, k, v, g, w.scale, causal))


def test_bwd_headline_shape_sampled_slices(osm):
    # The causal [2, 16, 4096, 128] workload (x8 query rows) at full size on
    # the GPU; the oracle recomputes two whole (b, h) slices.
    w = inputs.ATTN[inputs.HEADLINE_ATTN]
    q, k, v = inputs.attn_inputs(w)
    g = inputs.grad_output(q.shape, w.seed + 1)
    print(f"bwd {w.describe()}", flush=True)
    got = _gpu_bwd(osm, q, k, v, g, w.causal)
    for b, hh in ((0, 0), (w.B - 1, w.H - 1)):
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        ref = oracle.attn_bwd(q[sl], k[sl], v[sl], g[sl], w.scale, w.causal)
        _compare([x[sl] for x in got], ref, f"slice ({b}, {hh})",
                 _grad_bounds(q[sl], k[sl], v[sl], g[sl], w.scale, w.causal))


@pytest.mark.parametrize("case", [((1, 16, 2048, 64), False), ((1, 16, 2048, 64), True),
                                  ((1, 16, 2048, 128), False), ((1, 16, 2048, 128), True),
                                  ((2, 16, 2048, 64), False), ((2, 16, 2048, 64), True),
                                  ((2, 16, 2048, 128), False)])
def test_bwd_workgroup_sizes(osm, case):
    # The launch picks 8-, 4- or 2-wave workgroups for the dK/dV and dQ
    # kernels from how many it takes to cover the chip: [1, 16, 2048, d]
    # runs 4-wave workgroups (under both masks and at both head sizes),
    # [2, 16, 2048, d] 8-wave ones (d = 64 under both masks; d = 128 causal is
    # the headline test's).  The whole GPU problem, four whole (b, h) slices
    # recomputed by the oracle.
    (B, H, N, d), causal = case
    q, k, v, g = _case(B, H, N, d, seed=6000 + B * 7 + d)
    label = f"bwd B{B}H{H}N{N}d{d} causal={causal}"
    print(label, flush=True)
    got = _gpu_bwd(osm, q, k, v, g, causal)
    for bh in (0, 5, B * H - 6, B * H - 1):
        b, hh = divmod(bh, H)
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        ref = oracle.attn_bwd(q[sl], k[sl], v[sl], g[sl], 1.0 / math.sqrt(d), causal)
        _compare([x[sl] for x in got], ref, f"{label} slice ({b}, {hh})",
                 _grad_bounds(q[sl], k[sl], v[sl], g[sl], 1.0 / math.sqrt(d), causal))


def test_bwd_deterministic(osm):
    q, k, v, g = _case(1, 2, 1000, 128, seed=91)
    a = _gpu_bwd(osm, q, k, v, g, True)
    b = _gpu_bwd(osm, q, k, v, g, True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ----------------------------------------------------------- split backward --
def _gpu_bwd_split(osm, q, k, v, g, causal, nsplit):
    dev = torch.device("cuda:0")
    q, k, v, g = (t.to(dev) for t in (q, k, v, g))
    O, lse = osm.attention(q, k, v, causal=causal)
    dq, dk, dv = osm.attention_backward_split(q, k, v, O, lse, g, causal=causal, nsplit=nsplit)
    torch.cuda.synchronize()
    return [t.to(torch.float64).cpu().numpy() for t in (dq, dk, dv)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,nsplit", [((1, 2, 1000, 64), 3), ((1, 1, 777, 128), 4),
                                          ((2, 1, 512, 128), 2), ((1, 2, 1500, 128), 16),
                                          ((1, 1, 300, 64), 64)])
def test_bwd_split_full(osm, shape, nsplit, causal):
    # attn_bwd_split: the dK/dV query loop and the dQ key loop cut into
    # nsplit ranges, the fp32 partials summed.  Ragged N (a partial last
    # tile in every loop), uneven ranges, and more ranges than tiles (the
    # empty ranges contribute zeros).  Whole tensors against the oracle.
    B, H, N, d = shape
    q, k, v, g = _case(B, H, N, d, seed=7000 + N + d + nsplit)
    label = f"bwd split={nsplit} B{B}H{H}N{N}d{d} causal={causal}"
    print(label, flush=True)
    got = _gpu_bwd_split(osm, q, k, v, g, causal, nsplit)
    ref = oracle.attn_bwd(q, k, v, g, 1.0 / math.sqrt(d), causal)
    _compare(got, ref, label, _grad_bounds(q, k, v, g, 1.0 / math.sqrt(d), causal))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_split_gqa(osm, causal):
    # Four query heads on two key/value heads: a dK/dV workgroup's ranges run
    # over the query tiles of both heads of its group, head by head.
    B, H, Hkv, N, d = 1, 4, 2, 600, 128
    q, k, v, g = _case(B, H, N, d, seed=7100)
    k, v = k[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    label = f"bwd split=3 GQA B{B}H{H}/{Hkv}N{N}d{d} causal={causal}"
    print(label, flush=True)
    got = _gpu_bwd_split(osm, q, k, v, g, causal, 3)
    G = H // Hkv
    kr, vr = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    rq, rk, rv = oracle.attn_bwd(q, kr, vr, g, 1.0 / math.sqrt(d), causal)
    rk = rk.reshape(B, Hkv, G, N, d).sum(axis=2)
    rv = rv.reshape(B, Hkv, G, N, d).sum(axis=2)
    _compare(got, (rq, rk, rv), label)


def test_bwd_split_small_grid_full(osm):
    # A small grid at full length: [1, 2, 4096, 128] causal, the library's
    # own split count, every element against the oracle; and the same call
    # twice gives the same bits (partials summed in range order).
    osm_abi = osm
    B, H, N, d = 1, 2, 4096, 128
    ns, _ = osm_abi.attn_bwd_split_plan(B, H, H, N, d, True, 0)
    assert ns > 1
    q, k, v, g = _case(B, H, N, d, seed=7200)
    label = f"bwd split={ns} B{B}H{H}N{N}d{d} causal=True"
    print(label, flush=True)
    got = _gpu_bwd_split(osm, q, k, v, g, True, 0)
    ref = oracle.attn_bwd(q, k, v, g, 1.0 / math.sqrt(d), True)
    _compare(got, ref, label, _grad_bounds(q, k, v, g, 1.0 / math.sqrt(d), True))
    again = _gpu_bwd_split(osm, q, k, v, g, True, 0)
    assert all(np.array_equal(x, y) for x, y in zip(got, again))


def test_bwd_split_one_is_attn_bwd(osm):
    # A count of 1 is attn_bwd itself: bitwise the same gradients.
    q, k, v, g = _case(1, 2, 1000, 64, seed=7300)
    a = _gpu_bwd_split(osm, q, k, v, g, True, 1)
    b = _gpu_bwd(osm, q, k, v, g, True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
