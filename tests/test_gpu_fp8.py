"""GPU parity of the fp8 attention forward (attn_fwd_fp8 through the C ABI)
against the fp64 oracle on the decoded, scaled fp8 inputs, element by
element within the error contract of fp8_contract (the score summation of
the fp8 matrix cores, the rounding of the probabilities to fp8 and of O to
bf16); test_fp8_score_sum_error measures the summation error that contract
assumes.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu

from fp8_contract import EPS_S, _bars  # noqa: E402


@pytest.fixture(scope="module")
def osm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_08_amd
    return online_softmax_08_amd


def _gpu(osm, q8, k8, v8, sc, causal, scale):
    dev = torch.device("cuda:0")
    O, lse = osm.attention_fp8(q8.to(dev), k8.to(dev), v8.to(dev), *sc, causal=causal,
                               scale=scale)
    torch.cuda.synchronize()
    return O.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def _check(osm, q8, k8, v8, sc, causal, label, slices=None):
    B, H, N, d = q8.shape
    Hkv = k8.shape[1]
    G = H // Hkv
    scale = 1.0 / math.sqrt(d)
    O, lse = _gpu(osm, q8, k8, v8, sc, causal, scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse)), label
    worst, worst_lse = 0.0, 0.0
    for (b, hh) in (slices or [(b, hh) for b in range(B) for hh in range(H)]):
        qs, ks, vs = q8[b:b + 1, hh:hh + 1], k8[b:b + 1, hh // G:hh // G + 1], v8[b:b + 1, hh // G:hh // G + 1]
        Oref, lref = oracle.attn_fwd_fp8(qs, ks, vs, *sc, scale, causal)
        Qd, Kd, Vd = (oracle.fp8_decode(t, s)[0, 0] for t, s in zip((qs, ks, vs), sc))
        o_bar, lse_bar = _bars(Qd, Kd, Vd, scale, causal)
        r = np.abs(O[b, hh] - Oref[0, 0]) / o_bar
        rl = np.abs(lse[b, hh] - lref[0, 0]) / lse_bar
        worst = max(worst, float(r.max()) if r.size else 0.0)
        worst_lse = max(worst_lse, float(rl.max()) if rl.size else 0.0)
    print(f"{label}: max err/elem-bar O {worst:.3f} lse {worst_lse:.3f}", flush=True)
    assert worst <= 1.0 and worst_lse <= 1.0, label


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1000, 64), (2, 1, 777, 128), (1, 1, 65, 128),
                                   (1, 3, 1, 64), (1, 2, 256, 128), (1, 1, 300, 64)])
def test_fp8_full(osm, shape, causal):
    # Ragged N (partial last tiles, the causal diagonal in the last tile),
    # both head sizes, one-row and one-block problems; every element.
    B, H, N, d = shape
    w = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    (q8, k8, v8), sc = inputs.attn_inputs_fp8(w, B=B, H=H, N=N, d=d, seed=8000 + N + d)
    _check(osm, q8, k8, v8, sc, causal, f"fp8 B{B}H{H}N{N}d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_grouped_heads(osm, causal):
    # Four query heads on two key/value heads.
    w = inputs.ATTN["attn_bf16_B4H16N2048d128"]
    (q8, k8, v8), sc = inputs.attn_inputs_fp8(w, B=2, H=4, N=600, d=128, seed=8100, Hkv=2)
    _check(osm, q8, k8, v8, sc, causal, f"fp8 GQA B2H4/2N600d128 causal={causal}")


@pytest.mark.parametrize("shape", [(2, 16, 4096, 128), (2, 16, 4000, 128), (2, 16, 4000, 64)])
def test_fp8_large_sampled_slices(osm, shape):
    # The headline workload's shape and recipe (every 64th query row x8,
    # causal), stored as fp8, and ragged N at both head sizes: the whole GPU
    # problem, with four whole (b, h) slices recomputed by the oracle.
    B, H, N, d = shape
    w = inputs.ATTN[inputs.HEADLINE_ATTN]
    (q8, k8, v8), sc = inputs.attn_inputs_fp8(w, B=B, H=H, N=N, d=d)
    _check(osm, q8, k8, v8, sc, True, f"fp8 B{B}H{H}N{N}d{d} causal x8 rows",
           slices=[(0, 0), (0, 7), (1, 9), (1, 15)])


def test_fp8_deterministic(osm):
    w = inputs.ATTN["attn_bf16_B4H16N2048d128"]
    (q8, k8, v8), sc = inputs.attn_inputs_fp8(w, B=1, H=2, N=700, d=128, seed=8200)
    a = _gpu(osm, q8, k8, v8, sc, True, 0.1)
    b = _gpu(osm, q8, k8, v8, sc, True, 0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_sum_error(osm, d):
    # The score error the bars assume, measured through the public call: with
    # one key per row the logsumexp is the score itself (the reference moves
    # to it on tile 0, p' = 16 exactly), so lse - scale * q.k (exact, fp64) is
    # the matrix cores' summation error of one d-term dot product.  Gaussian
    # data (every 8th row x8) stored as E4M3 with per-tensor scales, 8192 rows.
    B, H, N = 1, 8192, 1
    g = torch.Generator().manual_seed(8300 + d)
    q = torch.randn((B, H, N, d), generator=g)
    k = torch.randn((B, H, N, d), generator=g)
    q[:, ::8] *= 8
    (q8, qs), (k8, ks) = inputs.fp8_quantize(q), inputs.fp8_quantize(k)
    v8 = torch.zeros_like(k8)
    scale = 1.0 / math.sqrt(d)
    _, lse = _gpu(osm, q8, k8, v8, (qs, ks, 1.0), False, scale)
    Qd, Kd = oracle.fp8_decode(q8, qs)[0, :, 0], oracle.fp8_decode(k8, ks)[0, :, 0]
    exact = scale * np.sum(Qd * Kd, axis=1)
    absum = scale * np.sum(np.abs(Qd * Kd), axis=1)
    r = np.abs(lse[0, :, 0] - exact) / absum
    print(f"d={d}: score error / (scale sum|q k|): median {np.median(r):.2e} max {r.max():.2e} "
          f"(bar EPS_S = {EPS_S:.2e})", flush=True)
    assert r.max() <= EPS_S
