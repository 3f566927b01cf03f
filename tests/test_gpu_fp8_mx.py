"""GPU parity of the block-quantized FP8 path ("Moving less", section 4.6:
block quantization and incoherent processing) through the C ABI:

* fp8_quantize_rows / fp8_quantize_cols against the oracle's block
  quantization: bit for bit without the rotation (the kernel takes every
  decision on the exact bf16 values, as the oracle does; +0 and -0 count as
  one code).  With the rotation the kernel forms the rotated values in fp32
  and the oracle in fp64, so a decision may differ where the exact value sits
  within the fp32 transform's error of a decision boundary: a scale where the
  block maximum is that close to 448 * 2^k, a code where the scaled value is
  that close to the midpoint of two codes.  Everything else must match, and
  the exempt cases must be rare and each one of the two valid choices.
* attn_fwd_fp8_mx against the oracle's attention on the values the
  oracle-quantized codes and scales stand for, element by element within the
  fp8 error contract of fp8_contract.
* The FP8 section's accuracy claim on the GPU path: with outlier channels in
  Q and K, block scales after the random-sign Hadamard rotation give O a
  much lower RMSE than one scale per tensor.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu

from fp8_contract import _bars  # noqa: E402


@pytest.fixture(scope="module")
def osm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_08_amd
    return online_softmax_08_amd


def _np(t):
    return t.cpu().numpy()


def _zero_same(c):
    """Codes with -0 (0x80) read as +0."""
    c = np.asarray(c, dtype=np.uint8)
    return np.where(c == 0x80, 0, c)


@pytest.mark.parametrize("shape", [(1, 2, 45, 64), (2, 3, 257, 128), (1, 1, 1, 128),
                                   (1, 1, 1000, 64)])
def test_quantize_rows_exact(osm, shape):
    B, H, N, d = shape
    q, _, _ = inputs.attn_inputs_blockwise(B=B, H=H, N=N, d=d, seed=9000 + N)
    codes, scales = osm.quantize_fp8_rows(q.cuda())
    torch.cuda.synchronize()
    oc, osc = oracle.mx_quantize_rows(q)
    np.testing.assert_array_equal(_np(scales), osc)
    np.testing.assert_array_equal(_zero_same(_np(codes)), _zero_same(oc))


@pytest.mark.parametrize("shape", [(1, 2, 45, 64), (2, 1, 1000, 128), (1, 3, 33, 128),
                                   (1, 1, 1, 64)])
def test_quantize_cols_exact(osm, shape):
    B, H, N, d = shape
    _, _, v = inputs.attn_inputs_blockwise(B=B, H=H, N=N, d=d, seed=9100 + N)
    codes, scales = osm.quantize_fp8_cols(v.cuda())
    torch.cuda.synchronize()
    oc, osc = oracle.mx_quantize_cols(v)
    assert scales.shape == (B, H, (N + 31) // 32, d)
    np.testing.assert_array_equal(_np(scales), osc)
    np.testing.assert_array_equal(_zero_same(_np(codes)), _zero_same(oc))


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_extreme_magnitudes(osm, d):
    # Blocks near the top of the bf16 range (2^125), tiny normals (2^-120),
    # bf16 subnormals (2^-130, whose scale byte clamps at 0 = 2^-127), mixed
    # blocks and exact zeros: scales and codes bit for bit, rows and columns.
    g = torch.Generator().manual_seed(9150 + d)
    x = torch.randn((1, 1, 64, d), generator=g)
    mags = [2.0 ** 125, 2.0 ** -120, 2.0 ** -130, 1.0, 0.0, 2.0 ** 100, 2.0 ** -133, 3.0]
    for r in range(64):
        x[0, 0, r] *= mags[r % len(mags)]
    x[0, 0, 3, :16] *= 2.0 ** -20  # a block mixing two magnitudes
    x = x.to(torch.bfloat16)
    codes, scales = osm.quantize_fp8_rows(x.cuda())
    vcodes, vscales = osm.quantize_fp8_cols(x.cuda())
    torch.cuda.synchronize()
    oc, osc = oracle.mx_quantize_rows(x)
    np.testing.assert_array_equal(_np(scales), osc)
    np.testing.assert_array_equal(_zero_same(_np(codes)), _zero_same(oc))
    vc, vsc = oracle.mx_quantize_cols(x)
    np.testing.assert_array_equal(_np(vscales), vsc)
    np.testing.assert_array_equal(_zero_same(_np(vcodes)), _zero_same(vc))


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_rows_rotated(osm, d):
    # Rows of the outlier recipe and of the block-scale recipe, rotated.
    qa, ka, _ = inputs.attn_inputs_outliers(B=1, H=2, N=700, d=d, seed=9200 + d)
    qb, _, _ = inputs.attn_inputs_blockwise(B=1, H=2, N=700, d=d, seed=9300 + d)
    x = torch.cat([qa, ka, qb], dim=1).contiguous()
    signs = inputs.hadamard_signs(d, seed=9400 + d)
    codes, scales = osm.quantize_fp8_rows(x.cuda(), signs)
    torch.cuda.synchronize()
    kc, ksc = _zero_same(_np(codes)), _np(scales).astype(np.int64)
    X = x.to(torch.float64).numpy()
    Y = oracle.hadamard_rotate(X, np.array(signs, dtype=np.float64))
    oc, osc = oracle.mx_quantize_rows(Y)
    oc, osc = _zero_same(oc), osc.astype(np.int64)
    rows = Y.reshape(-1, d)
    # The fp32 transform's error bound per row: log2(d) + 2 roundings of
    # size 2^-24 of sum_t |x_t| / sqrt(d), with a factor 4 to spare.
    slack = 4 * (math.log2(d) + 2) * 2.0 ** -24 * np.abs(X.reshape(-1, d)).sum(axis=1) / math.sqrt(d)
    blk = rows.reshape(rows.shape[0], d // 32, 32)
    amax = np.abs(blk).max(axis=2)
    ks, os_ = ksc.reshape(amax.shape), osc.reshape(amax.shape)
    bad_s = ks != os_
    lo = np.minimum(ks, os_) - 127
    near_b = np.abs(amax - 448.0 * np.exp2(lo)) <= slack[:, None]
    assert np.all(near_b[bad_s]) and np.all(np.abs(ks - os_)[bad_s] <= 1)
    # codes of blocks with equal scales
    kcb, ocb = kc.reshape(blk.shape), oc.reshape(blk.shape)
    same = ~bad_s
    diff = (kcb != ocb) & same[:, :, None]
    e = (os_ - 127)[:, :, None]
    kd = oracle.fp8_decode(kcb) * np.exp2(e)
    od = oracle.fp8_decode(ocb) * np.exp2(e)
    mid = 0.5 * (kd + od)
    near_m = np.abs(blk - mid) <= slack[:, None, None]
    step_ok = np.abs(kcb.astype(np.int64) - ocb.astype(np.int64)) == 1
    assert np.all(near_m[diff] & step_ok[diff]), "a code differs away from a rounding midpoint"
    # blocks whose scales differ: the kernel's codes are still nearest on its own grid
    if bad_s.any():
        ek = (ks - 127)[:, :, None]
        kdd = oracle.fp8_decode(kcb) * np.exp2(ek)
        half_step = np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * np.exp2(ek))
        err = np.abs(kdd - blk)
        assert np.all(err[np.broadcast_to(bad_s[:, :, None], err.shape)]
                      <= (half_step + slack[:, None, None])[np.broadcast_to(bad_s[:, :, None], err.shape)])
    n_ex = int(bad_s.sum()) + int(diff.sum())
    print(f"d={d}: {n_ex} exempt decisions of {kc.size + ks.size}", flush=True)
    assert n_ex <= 1e-4 * kc.size


def _mx_inputs(B, H, N, d, seed, Hkv=None, rotate=False):
    """Oracle-quantized inputs: codes and scales of Q, K (rows, after the
    oracle's rotation when asked) and V (columns) as CPU tensors."""
    q, k, v = inputs.attn_inputs_blockwise(B=B, H=H, N=N, d=d, seed=seed, Hkv=Hkv)
    Q, K = q.to(torch.float64).numpy(), k.to(torch.float64).numpy()
    if rotate:
        s = np.array(inputs.hadamard_signs(d, seed=seed + 1), dtype=np.float64)
        Q, K = oracle.hadamard_rotate(Q, s), oracle.hadamard_rotate(K, s)
    (q8, qs), (k8, ks) = oracle.mx_quantize_rows(Q), oracle.mx_quantize_rows(K)
    v8, vs = oracle.mx_quantize_cols(v)
    return tuple(torch.from_numpy(np.ascontiguousarray(a)) for a in (q8, qs, k8, ks, v8, vs))


def _check(osm, t, causal, label, slices=None):
    q8, qs, k8, ks, v8, vs = t
    B, H, N, d = q8.shape
    G = H // k8.shape[1]
    scale = 1.0 / math.sqrt(d)
    O, lse = osm.attention_fp8_mx(*(a.cuda() for a in t), causal=causal, scale=scale)
    torch.cuda.synchronize()
    O, lse = O.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse)), label
    worst, worst_lse = 0.0, 0.0
    for (b, hh) in (slices or [(b, hh) for b in range(B) for hh in range(H)]):
        kv = hh // G
        sl = (q8[b:b + 1, hh:hh + 1], qs[b:b + 1, hh:hh + 1], k8[b:b + 1, kv:kv + 1],
              ks[b:b + 1, kv:kv + 1], v8[b:b + 1, kv:kv + 1], vs[b:b + 1, kv:kv + 1])
        Oref, lref = oracle.attn_fwd_fp8_mx(*sl, scale, causal)
        Qd = oracle.mx_decode_rows(sl[0], sl[1])[0, 0]
        Kd = oracle.mx_decode_rows(sl[2], sl[3])[0, 0]
        Vd = oracle.mx_decode_cols(sl[4], sl[5])[0, 0]
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
def test_fp8_mx_full(osm, shape, causal):
    # Every block with its own scale (powers of two from 2^-4 to 2^4, some
    # blocks zero), ragged N, both head sizes, one-row and one-block problems.
    B, H, N, d = shape
    _check(osm, _mx_inputs(B, H, N, d, seed=9500 + N + d), causal,
           f"mx B{B}H{H}N{N}d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_mx_grouped_heads(osm, causal):
    _check(osm, _mx_inputs(2, 4, 600, 128, seed=9600, Hkv=2), causal,
           f"mx GQA B2H4/2N600d128 causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_mx_rotated_inputs(osm, d):
    # Q and K rotated by the oracle before quantizing: same contract on the
    # values the codes stand for.
    _check(osm, _mx_inputs(1, 2, 700, d, seed=9700 + d, rotate=True), True,
           f"mx rotated B1H2N700d{d} causal")


@pytest.mark.parametrize("shape", [(2, 16, 4096, 128), (1, 8, 4000, 64)])
def test_fp8_mx_large_sampled_slices(osm, shape):
    # The headline workload's size (and a ragged d = 64 one), causal, with
    # four whole (b, h) slices recomputed by the oracle.
    B, H, N, d = shape
    _check(osm, _mx_inputs(B, H, N, d, seed=9800 + d), True, f"mx B{B}H{H}N{N}d{d} causal",
           slices=[(0, 0), (0, H // 2 - 1), (B - 1, H // 2), (B - 1, H - 1)])


def test_fp8_mx_deterministic(osm):
    t = [a.cuda() for a in _mx_inputs(1, 2, 700, 128, seed=9900)]
    a = osm.attention_fp8_mx(*t, causal=True)
    b = osm.attention_fp8_mx(*t, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_block_outliers(osm):
    # The FP8 section's claim, end to end on the GPU path: Q and K with four
    # outlier head channels (x20).  One scale per tensor (attn_fwd_fp8 on
    # per-tensor codes) against block scales after the random-sign Hadamard
    # rotation (fp8_quantize_rows with signs, fp8_quantize_cols,
    # attn_fwd_fp8_mx), both against exact attention on the bf16 inputs.  The
    # pages report a 2.6x lower RMSE on their outlier test; here at least 2x.
    B, H, N, d = 1, 4, 1024, 128
    q, k, v = inputs.attn_inputs_outliers(B=B, H=H, N=N, d=d, seed=9950)
    scale = 1.0 / math.sqrt(d)
    Oref, _ = oracle.attn_fwd(q, k, v, scale, False)
    (q8, qs), (k8, ks), (v8, vs) = (inputs.fp8_quantize(t.to(torch.float32)) for t in (q, k, v))
    Ot, _ = osm.attention_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs, ks, vs, scale=scale)
    signs = inputs.hadamard_signs(d, seed=9951)
    Or, _ = osm.attention_fp8_block(q.cuda(), k.cuda(), v.cuda(), signs, scale=scale)
    Ob, _ = osm.attention_fp8_block(q.cuda(), k.cuda(), v.cuda(), None, scale=scale)
    Obf, _ = osm.attention(q.cuda(), k.cuda(), v.cuda(), scale=scale)
    torch.cuda.synchronize()

    def rmse(O):
        return float(np.sqrt(np.mean((O.to(torch.float64).cpu().numpy() - Oref) ** 2)))
    rt, rr, rb, rbf = rmse(Ot), rmse(Or), rmse(Ob), rmse(Obf)
    print(f"RMSE of O: per-tensor fp8 {rt:.3e}, block fp8 {rb:.3e}, "
          f"block fp8 + rotation {rr:.3e}, bf16 {rbf:.3e}", flush=True)
    assert rr * 2.0 < rt
