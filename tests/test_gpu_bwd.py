"""GPU parity of the attention backward (dQ, dK, dV through the C ABI)
against the fp64 oracle's chain-rule gradients, on seeded inputs.

The GPU backward takes the forward's own bf16 O and fp32 lse as inputs, as a
training step would; the oracle recomputes everything from Q, K, V and dO in
fp64.  Bar, per gradient tensor: max-abs error <= 2e-2 * max(1, max |ref|),
i.e. the forward's bf16 bar for gradients up to 1 and 2% of the tensor's
largest magnitude beyond.  The error is not a fixed multiple of one bf16
rounding: D_i = sum_t dO_it O_it is formed from the rounded O (relative error
up to 2^-9 per term), and that error reaches dK_j through
scale * sum_i P_ij dD_i Q_i, which the x8 query rows of the causal stress
workload amplify (there it is 0.10 of the 0.13 max error on dK, |dK| <= 14);
the bf16 rounding of P and dS inside the products adds the rest.
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


def _compare(got, ref, label):
    ok = True
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(a)), f"{label}: {name} not finite"
        e = float(np.max(np.abs(a - b))) if a.size else 0.0
        scale = max(1.0, float(np.max(np.abs(b))) if b.size else 0.0)
        print(f"{label}: {name} max|err|={e:.3e} max|ref|={scale:.3f} bar={TOL * scale:.3e}", flush=True)
        ok &= e <= TOL * scale
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
    _compare(got, ref, label)


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
    _compare(got, ref, label)


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
        _compare([x[sl] for x in got], ref, f"slice ({b}, {hh})")


@pytest.mark.parametrize("case", [((1, 16, 2048, 64), False), ((1, 16, 2048, 64), True),
                                  ((1, 16, 2048, 128), False), ((1, 16, 2048, 128), True),
                                  ((2, 16, 2048, 64), False), ((2, 16, 2048, 128), False)])
def test_bwd_workgroup_sizes(osm, case):
    # The launch picks 8-, 4- or 2-wave workgroups for the dK/dV and dQ
    # kernels from how many it takes to cover the chip: [1, 16, 2048, d]
    # runs 4-wave workgroups (under both masks and at both head sizes),
    # [2, 16, 2048, d] unmasked 8-wave ones.  The whole GPU problem, four
    # whole (b, h) slices recomputed by the oracle.
    (B, H, N, d), causal = case
    q, k, v, g = _case(B, H, N, d, seed=6000 + B * 7 + d)
    label = f"bwd B{B}H{H}N{N}d{d} causal={causal}"
    print(label, flush=True)
    got = _gpu_bwd(osm, q, k, v, g, causal)
    for bh in (0, 5, B * H - 6, B * H - 1):
        b, hh = divmod(bh, H)
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        ref = oracle.attn_bwd(q[sl], k[sl], v[sl], g[sl], 1.0 / math.sqrt(d), causal)
        _compare([x[sl] for x in got], ref, f"{label} slice ({b}, {hh})")


def test_bwd_deterministic(osm):
    q, k, v, g = _case(1, 2, 1000, 128, seed=91)
    a = _gpu_bwd(osm, q, k, v, g, True)
    b = _gpu_bwd(osm, q, k, v, g, True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
