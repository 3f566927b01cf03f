"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element.

Tolerances (max-abs over every compared element): fp32 paths 1e-5 on O, lse
and softmax outputs; bf16 attention 2e-2 on O and 1e-3 on lse.  Every
workload is compared in full, the large ones at full size in the launch
configuration the benchmark times, plus properties that hold at any size.
Sweeps whose only purpose is to reach each launch configuration compare
sampled rows.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(scope="module")
def osm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_08_amd
    return online_softmax_08_amd


def _gpu_attn(osm, q, k, v, causal, scale=None):
    dev = torch.device("cuda:0")
    O, lse = osm.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return O.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def _maxabs(a, b):
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def _check_full(osm, q, k, v, causal, dtype, label, scale=None):
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    O, lse = _gpu_attn(osm, q, k, v, causal, scale)
    Oref, lref = oracle.attn_fwd(q, k, v, scale, causal)
    eo, el = _maxabs(O, Oref), _maxabs(lse, lref)
    to, tl = TOL[dtype]
    print(f"{label}: max|dO|={eo:.3e} (tol {to}) max|dlse|={el:.3e} (tol {tl})", flush=True)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    assert eo <= to and el <= tl, label
    return O, lse


def _sample_rows(w, rng, n_slices=8, n_random=16):
    BH, N = w.B * w.H, w.N
    slices = sorted({0, BH - 1, *rng.choice(BH, size=min(BH, n_slices - 2), replace=False).tolist()})
    fixed = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 255, 256, 257, N // 2, N - 65, N - 64, N - 2, N - 1]
    bh, qi = [], []
    for s in slices:
        rows = sorted({r for r in fixed if 0 <= r < N} |
                      set(rng.choice(N, size=n_random, replace=False).tolist()))
        bh += [s] * len(rows)
        qi += rows
    return np.array(bh), np.array(qi)


# ----------------------------------------------------------------- attention --

@pytest.mark.parametrize("name", ["attn_f32_B1H1N128d64", "attn_bf16_B2H8N1024d64"])
def test_attn_workload_full(osm, name):
    w = inputs.ATTN[name]
    q, k, v = inputs.attn_inputs(w)
    print(w.describe(), flush=True)
    _check_full(osm, q, k, v, w.causal, w.dtype, name)


@pytest.mark.parametrize("name", ["attn_bf16_B4H16N2048d128",
                                  "attn_bf16_B2H16N4096d128_causal_x8rows",
                                  "attn_bf16_B1H32N8192d128_causal"])
def test_attn_workload_large_full(osm, name):
    # The three large workloads in the launch configuration the benchmark
    # times, every element compared with the oracle (a few seconds of host
    # work each), plus the convex-hull property: every output row is a convex
    # combination of value rows, so it lies within each column's [min, max].
    w = inputs.ATTN[name]
    print(w.describe(), flush=True)
    q, k, v = inputs.attn_inputs(w)
    O, lse = _check_full(osm, q, k, v, w.causal, w.dtype, name, w.scale)
    vf = v.to(torch.float32)
    lo = vf.amin(dim=2, keepdim=True).numpy() - 2e-2
    hi = vf.amax(dim=2, keepdim=True).numpy() + 2e-2
    assert np.all(O >= lo) and np.all(O <= hi)


@pytest.mark.parametrize("shape", [(2, 16, 4000, 64), (2, 16, 4096, 64), (2, 16, 4000, 128)])
def test_attn_phase_staggered_causal_full(osm, shape):
    # 512 query blocks of 256 rows: the phase-staggered kernel under the
    # causal mask, at d = 64 (its own tile-load schedule: V loads issued in
    # the vector phase) and with a ragged N (4000 = 15 full blocks plus 160
    # rows; the last block's diagonal tile is also the tail tile).  Every
    # element against the oracle.
    B, H, N, d = shape
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q, k, v = inputs.attn_inputs(base, B=B, H=H, N=N, d=d, seed=base.seed + 31 * N + d)
    _check_full(osm, q, k, v, True, "bf16", f"phase-staggered causal B{B}H{H}N{N}d{d}")


EDGE_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_attn_edge_shapes(osm, dtype, d, causal):
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if dtype == "bf16" else "attn_f32_B1H1N128d64"]
    for N in EDGE_N:
        q, k, v = inputs.attn_inputs(base, B=1, H=2, N=N, d=d, seed=base.seed + 1000 + N)
        _check_full(osm, q, k, v, causal, dtype, f"{dtype} d={d} causal={causal} N={N}")


def test_attn_multi_batch_head_slices(osm):
    # Odd B and H; each slice must match the oracle (no cross-slice mixing).
    base = inputs.ATTN["attn_bf16_B2H8N1024d64"]
    for d in (64, 128):
        q, k, v = inputs.attn_inputs(base, B=3, H=5, N=200, d=d, seed=77)
        for causal in (False, True):
            _check_full(osm, q, k, v, causal, "bf16", f"B3H5N200 d={d} causal={causal}")


def test_attn_rescale_stress(osm):
    # Scores that rise along the keys force the running maximum to move on every
    # tile (the rescale path); the first query row's boosted copy gives huge
    # logits.  Built from grid values so the bf16 inputs are exact.
    N, d = 700, 128
    q = torch.zeros(1, 2, N, d)
    k = torch.zeros(1, 2, N, d)
    q[..., 0] = 1.0
    q[:, 1, ::7, 0] = 16.0
    k[..., 0] = torch.arange(N, dtype=torch.float32) / 32.0
    g = torch.Generator().manual_seed(5)
    v = torch.randn(1, 2, N, d, generator=g)
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    for causal in (False, True):
        _check_full(osm, q, k, v, causal, "bf16", f"rising scores causal={causal}")
        _check_full(osm, q.float(), k.float(), v.float(), causal, "f32",
                    f"rising scores f32 causal={causal}")


def test_attn_rescale_stress_full_grid(osm):
    # Scores built to move the exponent reference in every way, on a grid
    # large enough for the phase-staggered kernel under both masks (512
    # query blocks of 256 rows).
    # Eight kinds of head (score = q_0 k_0 plus small noise): keys rising by
    # 12, 2 or 0.16 (log2 units) per 64-key tile, rising by 13 per tile for
    # queries boosted x16, falling scores, and jumps of ~150 log2 units in
    # mid-tile or at a tile boundary, where every probability of the tile
    # overflows against the old reference and must be recomputed.  Scaled
    # scores stay below ~150 so that fp32 resolves lse to 1e-3.  Every row of
    # the eight head kinds is compared with the oracle.
    B, H, N, d = 1, 128, 1024, 128
    j = torch.arange(N, dtype=torch.float32)
    kind = [1.5 * j, 0.25 * j, 0.1 * j, 1200.0 * (j >= 300), 1200.0 * (j >= 512), -0.5 * j,
            0.02 * j, 400.0 * (j >= 200) + 800.0 * (j >= 700)]
    qboost = [1.0, 1.0, 16.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    g = torch.Generator().manual_seed(15)
    q = 0.25 * torch.randn(B, H, N, d, generator=g)
    k = 0.25 * torch.randn(B, H, N, d, generator=g)
    v = torch.randn(B, H, N, d, generator=g)
    for h in range(H):
        q[0, h, :, 0] = qboost[h % 8]
        k[0, h, :, 0] = kind[h % 8]
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    scale = 1.0 / math.sqrt(d)
    heads = list(range(8)) + [45, 127]
    bh = np.repeat(np.array(heads), N)
    qi = np.tile(np.arange(N), len(heads))
    for causal in (False, True):
        O, lse = _gpu_attn(osm, q, k, v, causal, scale)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
        Oref, lref = oracle.attn_rows(q, k, v, scale, causal, bh, qi)
        eo = _maxabs(O.reshape(B * H, N, d)[bh, qi], Oref)
        el = _maxabs(lse.reshape(B * H, N)[bh, qi], lref)
        print(f"rescale stress, 8-wave grid, causal={causal}: max|dO|={eo:.3e} max|dlse|={el:.3e} "
              f"(max |lse| {np.max(np.abs(lref)):.1f})", flush=True)
        assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_attn_constant_values(osm):
    # All value rows equal to c: O must equal c (up to bf16 rounding of c's
    # products, here exact because p sums to 1 and c is a small grid value).
    base = inputs.ATTN["attn_bf16_B2H8N1024d64"]
    q, k, _ = inputs.attn_inputs(base, B=1, H=2, N=333, d=128, seed=9)
    c = torch.linspace(-2, 2, 128).bfloat16().float()
    v = c.expand(1, 2, 333, 128).contiguous().bfloat16()
    O, _ = _gpu_attn(osm, q, k, v, True, 1.0 / math.sqrt(128))
    assert _maxabs(O, np.broadcast_to(c.numpy(), O.shape)) <= 2e-2


def test_attn_deterministic(osm):
    w = inputs.ATTN["attn_bf16_B2H16N4096d128_causal_x8rows"]
    q, k, v = inputs.attn_inputs(w, B=1, H=4, N=1500)
    dev = torch.device("cuda:0")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    O1, l1 = osm.attention(q, k, v, causal=True)
    O2, l2 = osm.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 8, 2048, 64), (1, 16, 2048, 128), (1, 16, 3000, 64),
                                   (2, 16, 2048, 64), (2, 8, 4096, 128), (1, 2, 4096, 128)])
def test_attn_workgroup_sizes(osm, shape, causal):
    # The launch picks the workgroup shape from how many it takes to cover
    # the chip.  The 128-row workgroups of two key groups run (1, 16, 2048,
    # 128) and (2, 8, 2048, 64) under both masks, and the other shapes but
    # the last under the causal mask; the phase-staggered kernel runs those
    # without the mask (d = 64 and 128, ragged N = 3000); the 64-row
    # workgroups of two key groups run the last, at long N, for both masks.
    # Sampled rows against the oracle, every row finite.
    B, H, N, d = shape
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q, k, v = inputs.attn_inputs(base, B=B, H=H, N=N, d=d, seed=base.seed + 7 * N + d)
    scale = 1.0 / math.sqrt(d)
    O, lse = _gpu_attn(osm, q, k, v, causal, scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    w = inputs.AttnWorkload(name="wg", dtype="bf16", B=B, H=H, N=N, d=d, causal=causal, seed=base.seed)
    rng = np.random.default_rng(N + d + causal)
    bh, qi = _sample_rows(w, rng, n_slices=4, n_random=12)
    Oref, lref = oracle.attn_rows(q, k, v, scale, causal, bh, qi)
    eo = _maxabs(O.reshape(B * H, N, d)[bh, qi], Oref)
    el = _maxabs(lse.reshape(B * H, N)[bh, qi], lref)
    print(f"B{B}H{H}N{N}d{d} causal={causal}: {len(qi)} rows max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_attn_custom_scale(osm):
    base = inputs.ATTN["attn_bf16_B2H8N1024d64"]
    q, k, v = inputs.attn_inputs(base, B=1, H=2, N=190, d=64, seed=3)
    for causal in (False, True):
        _check_full(osm, q, k, v, causal, "bf16", f"scale=0.3 causal={causal}", scale=0.3)


# ------------------------------------------------------------------- softmax --

def _gpu_softmax(osm, x, inplace=False, offset=0):
    dev = torch.device("cuda:0")
    if offset:
        # Shift the data by `offset` floats inside a larger buffer (misaligned rows).
        buf = torch.empty(x.numel() + offset, dtype=torch.float32, device=dev)
        xd = buf[offset:].view(x.shape)
        xd.copy_(x.to(dev))
    else:
        xd = x.to(dev)
    y = osm.softmax(xd, out=xd if inplace else None)
    torch.cuda.synchronize()
    return y.to(torch.float64).cpu().numpy()


def test_softmax_small_workload(osm):
    w = inputs.SOFTMAX["softmax_f32_4x128"]
    x = inputs.softmax_inputs(w)
    y = _gpu_softmax(osm, x)
    e = _maxabs(y, oracle.row_softmax(x))
    print(f"{w.describe()}: max|dy|={e:.3e}", flush=True)
    assert np.all(np.isfinite(y)) and e <= 1e-5


def test_softmax_large_workload(osm):
    # Every element of the [32768, 8192] workload against the oracle, and
    # every row sums to 1.
    w = inputs.SOFTMAX["softmax_f32_32768x8192"]
    x = inputs.softmax_inputs(w)
    dev = torch.device("cuda:0")
    y = osm.softmax(x.to(dev))
    torch.cuda.synchronize()
    s = y.double().sum(dim=1)
    assert torch.all(torch.isfinite(y)) and float((s - 1).abs().max()) <= 1e-5
    e = _maxabs(y.double().cpu().numpy(), oracle.row_softmax(x))
    print(f"{w.describe()}: all rows max|dy|={e:.3e}", flush=True)
    assert e <= 1e-5


SOFTMAX_N = [1, 2, 3, 4, 5, 63, 64, 65, 127, 128, 129, 1000, 1023, 1024, 1025, 2048, 3001,
             4096, 4097, 8192, 8193, 12000, 16384, 20000, 32768, 32769, 65536, 100003]


@pytest.mark.parametrize("N", SOFTMAX_N)
def test_softmax_edge_widths(osm, N):
    w = inputs.SOFTMAX["softmax_f32_4x128"]
    B = 5 if N <= 65536 else 2
    x = inputs.softmax_inputs(w, B=B, N=N, seed=w.seed + N)
    ref = oracle.row_softmax(x)
    for inplace, offset in ((False, 0), (True, 0), (False, 1)):
        y = _gpu_softmax(osm, x, inplace=inplace, offset=offset)
        e = _maxabs(y, ref)
        assert np.all(np.isfinite(y)) and e <= 1e-5, (N, inplace, offset, e)


def test_softmax_extreme_rows(osm):
    # Huge common offsets, a single dominant element, constant rows.
    N = 2000
    x = torch.zeros(4, N)
    x[0] = 1000.0 - torch.arange(N, dtype=torch.float32)
    x[1] = -1000.0 + torch.arange(N, dtype=torch.float32) * 0.5
    x[2, 123] = 80.0
    x[3] = 3.25
    y = _gpu_softmax(osm, x)
    e = _maxabs(y, oracle.row_softmax(x))
    assert np.all(np.isfinite(y)) and e <= 1e-5


@pytest.mark.parametrize("N", [3, 64])
def test_softmax_more_rows_than_one_dispatch(osm, N):
    # Rows go out in dispatches of 2^21 rows (the same loop for every row
    # length); rows on both sides of the boundary and a random sample
    # against the oracle, all rows finite.
    B = (1 << 21) + 77
    g = torch.Generator().manual_seed(N)
    x = torch.randn((B, N), generator=g) * 3.0
    y = _gpu_softmax(osm, x)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(N)
    rows = sorted({0, (1 << 21) - 2, (1 << 21) - 1, 1 << 21, (1 << 21) + 1, B - 1,
                   *rng.choice(B, size=32, replace=False).tolist()})
    e = _maxabs(y[rows], oracle.row_softmax(x[rows]))
    print(f"softmax B={B} N={N}: {len(rows)} rows max|dy|={e:.3e}", flush=True)
    assert e <= 1e-5
