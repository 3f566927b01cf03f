"""The allocation-free backward (attn_bwd_noalloc, row statistics in the
library's static device scratch) against attn_bwd with a caller workspace,
through the C ABI, on the same inputs: two calls in a row, the second with a
smaller problem, each bitwise equal to attn_bwd (the same kernels on the same
inputs) and within the backward's bar of the fp64 oracle on whole slices."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from online_softmax_08_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from online_softmax_08_amd import _abi
    return _abi


def _run(abi, B, H, Hkv, N, d, causal, seed):
    dev = torch.device("cuda:0")
    base = inputs.ATTN["attn_bf16_B2H8N1024d64" if d == 64 else "attn_bf16_B4H16N2048d128"]
    q = inputs.attn_inputs(base, B=B, H=H, N=N, d=d, seed=seed)[0]
    _, k, v = inputs.attn_inputs(base, B=B, H=Hkv, N=N, d=d, seed=seed + 1)
    g = inputs.grad_output(q.shape, seed + 2)
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    scale = 1.0 / math.sqrt(d)
    O = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    abi.attn_fwd_gqa(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), O.data_ptr(), lse.data_ptr(),
                     B, H, Hkv, N, d, scale, causal, stream)
    outs = {}
    for mode in ("workspace", "noalloc"):
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        if mode == "workspace":
            ws = torch.empty(abi.attn_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
            abi.attn_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), O.data_ptr(), gd.data_ptr(),
                         lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N,
                         d, scale, causal, ws.data_ptr(), ws.numel(), stream)
        else:
            abi.attn_bwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), O.data_ptr(),
                                 gd.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                 dv.data_ptr(), B, H, Hkv, N, d, scale, causal, stream)
        torch.cuda.synchronize()
        outs[mode] = (dq, dk, dv)
    return (q, k, v, g, scale), outs


def _check(abi, B, H, Hkv, N, d, causal, seed, oracle_slices=True):
    (q, k, v, g, scale), outs = _run(abi, B, H, Hkv, N, d, causal, seed)
    label = f"B{B}H{H}Hkv{Hkv}N{N}d{d} causal={causal}"
    print(label, flush=True)
    for name, a, b in zip(("dQ", "dK", "dV"), outs["noalloc"], outs["workspace"]):
        assert torch.equal(a, b), f"{label}: {name} differs from attn_bwd"
        assert bool(torch.isfinite(a.float()).all()), f"{label}: {name} not finite"
    if not oracle_slices:
        return
    # whole first and last (b, h) slices against the oracle (the backward bar)
    G = H // Hkv
    for b, hh in ((0, 0), (B - 1, H - 1)):
        kvh = hh // G
        ref = oracle.attn_bwd(q[b:b + 1, hh:hh + 1], k[b:b + 1, kvh:kvh + 1],
                              v[b:b + 1, kvh:kvh + 1], g[b:b + 1, hh:hh + 1], scale, causal)
        got = outs["noalloc"][0][b, hh].double().cpu().numpy()
        e = float(np.max(np.abs(got - ref[0][0, 0])))
        bar = 2e-2 * max(1.0, float(np.max(np.abs(ref[0]))))
        print(f"{label}: dQ slice ({b}, {hh}) max|err|={e:.3e} bar={bar:.3e}", flush=True)
        assert e <= bar


def test_noalloc_matches_workspace_backward_two_calls(abi):
    # A larger call, then a smaller one on the same scratch (which still
    # holds the first call's statistics beyond the second call's rows).
    _check(abi, 2, 16, 16, 2048, 128, True, seed=4100)
    _check(abi, 1, 4, 2, 333, 64, False, seed=4200)


def test_noalloc_at_the_row_limit(abi):
    # B * H * N exactly the scratch's limit (the statistics fill it; bitwise
    # against attn_bwd only, its slices are too long for the oracle), then a
    # small call again.
    rows = abi.NOALLOC_BWD_MAX_ROWS
    _check(abi, 1, 256, 256, rows // 256, 64, True, seed=4300, oracle_slices=False)
    _check(abi, 1, 2, 2, 100, 128, True, seed=4400)
