"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, never against the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with
  * a value a page prints for a worked example (tests/golden, with the page's
    title and section and a tolerance from its printed digits),
  * a closed form,
  * an invariant of softmax / attention,
  * an independent library routine (torch / scipy in float64), or
  * brute force on tiny inputs (the naive softmax without max subtraction,
    and the online recurrence against the three-pass definition).
``tests/test_oracle.py`` runs every pin on the committed oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in copies of the
oracle's C source and requires each to fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

_GOLDEN_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                            "worked_examples.json")
with open(_GOLDEN_PATH) as _f:
    GOLDEN = json.load(_f)


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a) == np.isfinite(b)), f"{what}: finiteness differs"
    fin = np.isfinite(a)
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    err = np.abs(a[fin] - b[fin])
    bound = atol + rtol * np.abs(b[fin])
    if err.size and not np.all(err <= bound):
        k = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: |{a[fin][k]} - {b[fin][k]}| = {err[k]:.3e} "
                             f"> {bound[k]:.3e}")


def _scores_as_attention(scores, values, causal=False):
    """A one-dimensional attention problem whose every query row sees the
    given scores: d = 1, scale = 1, q = 1, k_j = scores[j], v_j = values[j]."""
    n = len(scores)
    Q = np.ones((1, 1, n, 1))
    K = np.asarray(scores, dtype=np.float64).reshape(1, 1, n, 1)
    V = np.asarray(values, dtype=np.float64).reshape(1, 1, n, 1)
    return Q, K, V


def _rand_attn(rng, B, H, N, d, std=1.0):
    return (rng.standard_normal((B, H, N, d)) * std,
            rng.standard_normal((B, H, N, d)),
            rng.standard_normal((B, H, N, d)))


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

def pin_fusion_naive_three_keys(orc):
    g = GOLDEN["fusion_naive_three_keys"]
    p = orc.row_softmax(np.array([g["scores"]]))[0]
    _close(p, g["printed_probabilities"], g["prob_tol"], what="printed probabilities")
    Q, K, V = _scores_as_attention(g["scores"], g["values"])
    O, lse = orc.attn_fwd(Q, K, V, 1.0, False)
    _close(O[0, 0, :, 0], [g["printed_output"]] * 3, g["output_tol"],
           what="printed output")
    # Under the causal mask query 0 sees only key 0: its output is v_0 exactly.
    Oc, lsec = orc.attn_fwd(Q, K, V, 1.0, True)
    _close(Oc[0, 0, 0, 0], g["values"][0], 0.0, what="causal row 0")
    _close(lsec[0, 0, 0], g["scores"][0], 0.0, what="causal row 0 lse")
    # Query 2 sees every key, so it must match the non-causal row.
    _close(Oc[0, 0, 2, 0], O[0, 0, 2, 0], 1e-14, what="causal last row")


def pin_lesson22_two_blocks(orc):
    g = GOLDEN["lesson22_two_blocks_2_1_then_4_3"]
    m, l = orc.online_row_trace(g["scores"], g["block"])
    _close(m, g["printed_max_after_block"], 0.0, what="running max")
    e = math.e
    l1 = 1.0 + e ** -1                         # the page's expression for block 1
    l2 = e ** -2 * (1.0 + e ** -1) + 1.0 + e ** -1
    _close(l, [l1, l2], 0.0, 1e-15, what="running denominator")
    # The page notes the merged value equals the direct four-term sum, i.e. the
    # full-row denominator: lse of the three-pass definition is m + ln l.
    Q, K, V = _scores_as_attention(g["scores"], [1.0, 2.0, 3.0, 4.0])
    _, lse = orc.attn_fwd(Q, K, V, 1.0, False)
    _close(lse[0, 0, :], [4.0 + math.log(l2)] * 4, 0.0, 1e-15, what="lse")


def pin_fusion_two_blocks(orc):
    g = GOLDEN["fusion_two_blocks_2_1_then_4"]
    m, l = orc.online_row_trace(g["scores"], g["block"])
    _close(l[0], g["printed_sum_after_block1"], g["sum1_tol"], what="sum after block 1")
    # The correction factor is the ratio the old sum was scaled by; recover it
    # from the trace: l2 = c * l1 + (contribution of block 2, which is 1 here
    # because block 2 holds only the new maximum).
    corr = (l[1] - 1.0) / l[0]
    _close(corr, g["printed_correction"], g["corr_tol"], what="correction")
    _close(l[1], g["printed_sum_after_block2"], g["sum2_tol"], what="sum after block 2")


def pin_four_generations_blocks(orc):
    g = GOLDEN["four_generations_blocks_1_3_then_2_5"]
    m, l = orc.online_row_trace(g["scores"], g["block"])
    _close(m, g["printed_max_after_block"], 0.0, what="running max")
    _close(l, g["printed_sum_after_block"], g["sum_tol"], what="running denominator")
    # ... and the two-block result equals the one-shot row (three passes).
    Q, K, V = _scores_as_attention(g["scores"], [0.0] * 4)
    _, lse = orc.attn_fwd(Q, K, V, 1.0, False)
    _close(lse[0, 0, 0], m[-1] + math.log(l[-1]), 0.0, 1e-15, what="full-row lse")


def pin_overflow_row(orc):
    g = GOLDEN["lesson22_overflow_row"]
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(np.array(g["scores"])) / np.sum(np.exp(np.array(g["scores"])))
    assert np.all(np.isnan(naive)), "the naive formula should give inf/inf = NaN"
    p = orc.row_softmax(np.array([g["scores"], g["shift_equivalent"]]))
    assert np.all(np.isfinite(p)), "stable softmax must stay finite"
    _close(p[0], p[1], 0.0, 1e-15, what="shift invariance")
    # Closed form of softmax([2,1,0]) = e^{-j} / (1 + e^-1 + e^-2).
    z = 1.0 + math.exp(-1.0) + math.exp(-2.0)
    _close(p[0], [1.0 / z, math.exp(-1.0) / z, math.exp(-2.0) / z], 0.0, 1e-15,
           what="closed form")
    # The same row reversed and placed among small values: only subtracting the
    # true maximum (not, say, the first element) keeps every exponent <= 0.
    q = orc.row_softmax(np.array([[0.0, 998.0, 999.0, 1000.0, -5.0]]))[0]
    assert np.all(np.isfinite(q)), "stable softmax must stay finite"
    _close(q[1:4], p[0][::-1], 1e-300, 1e-13, what="reversed overflow row")


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_falling_row_closed_form(orc):
    # Row 1000 - j: a geometric sequence, p_j = e^{-j}(1 - e^-1)/(1 - e^-N).
    for n in (3, 128, 700):
        x = 1000.0 - np.arange(n, dtype=np.float64)
        p = orc.row_softmax(x[None, :])[0]
        j = np.arange(n, dtype=np.float64)
        ref = np.exp(-j) * (-math.expm1(-1.0)) / (-math.expm1(-float(n)))
        _close(p, ref, 1e-300, 1e-13, what=f"falling row N={n}")


def pin_two_element_logistic(orc):
    rng = _rng(11)
    ab = rng.standard_normal((64, 2)) * 10.0
    p = orc.row_softmax(ab)
    ref0 = 1.0 / (1.0 + np.exp(ab[:, 1] - ab[:, 0]))
    _close(p[:, 0], ref0, 0.0, 1e-14, what="logistic")
    _close(p[:, 1], 1.0 - ref0, 1e-15, 1e-13, what="logistic complement")


def pin_uniform_rows(orc):
    for n in (1, 2, 7, 4096):
        x = np.full((3, n), -3.25)
        p = orc.row_softmax(x)
        _close(p, np.full((3, n), 1.0 / n), 0.0, 1e-15, what=f"uniform N={n}")


def pin_attn_zero_keys(orc):
    rng = _rng(12)
    B, H, N, d = 2, 3, 37, 5
    Q, _, V = _rand_attn(rng, B, H, N, d)
    K = np.zeros_like(Q)
    O, lse = orc.attn_fwd(Q, K, V, 0.3, False)
    _close(O, np.broadcast_to(V.mean(axis=2, keepdims=True), O.shape), 1e-14,
           what="mean of V")
    _close(lse, np.full(lse.shape, math.log(N)), 1e-14, what="ln N")
    Oc, lsec = orc.attn_fwd(Q, K, V, 0.3, True)
    cum = np.cumsum(V, axis=2) / np.arange(1, N + 1).reshape(1, 1, N, 1)
    _close(Oc, cum, 1e-14, what="running mean of V")
    _close(lsec, np.broadcast_to(np.log(np.arange(1, N + 1.0)), lsec.shape), 1e-14,
           what="ln(i+1)")


def pin_attn_constant_values(orc):
    rng = _rng(13)
    B, H, N, d = 1, 2, 29, 6
    Q, K, _ = _rand_attn(rng, B, H, N, d, std=3.0)
    c = rng.standard_normal(d)
    V = np.broadcast_to(c, (B, H, N, d)).copy()
    for causal in (False, True):
        O, _ = orc.attn_fwd(Q, K, V, 0.5, causal)
        _close(O, V, 1e-14, 1e-14, what=f"constant V causal={causal}")


def pin_attn_causal_first_row_and_single_key(orc):
    rng = _rng(14)
    B, H, N, d = 2, 2, 9, 4
    Q, K, V = _rand_attn(rng, B, H, N, d)
    O, lse = orc.attn_fwd(Q, K, V, 0.7, True)
    _close(O[:, :, 0, :], V[:, :, 0, :], 0.0, what="causal row 0 output")
    dot0 = np.einsum("bhd,bhd->bh", Q[:, :, 0, :], K[:, :, 0, :])
    _close(lse[:, :, 0], 0.7 * dot0, 0.0, 1e-15, what="causal row 0 lse")
    for causal in (False, True):
        O1, lse1 = orc.attn_fwd(Q[:, :, :1], K[:, :, :1], V[:, :, :1], 0.7, causal)
        _close(O1, V[:, :, :1], 0.0, what="N=1 output")
        _close(lse1[:, :, 0], 0.7 * dot0, 0.0, 1e-15, what="N=1 lse")


# --------------------------------------------------------------------------
# Independent library routines (torch / scipy, float64)
# --------------------------------------------------------------------------

def pin_softmax_library(orc):
    import scipy.special
    import torch
    rng = _rng(15)
    for B, N, std in ((5, 1, 1.0), (7, 33, 4.0), (3, 1000, 30.0), (2, 8192, 1.0)):
        x = rng.standard_normal((B, N)) * std
        p = orc.row_softmax(x)
        _close(p, scipy.special.softmax(x, axis=1), 1e-300, 1e-12, what="scipy softmax")
        _close(p, torch.softmax(torch.from_numpy(x), dim=1).numpy(), 1e-300, 1e-12,
               what="torch softmax")


def _torch_attn(Q, K, V, scale, causal):
    import torch
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)) for a in (Q, K, V))
    O = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal,
                                                         scale=scale)
    S = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = S.shape[-1]
        S = S.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return O.numpy(), torch.logsumexp(S, dim=-1).numpy()


def pin_attn_library(orc):
    rng = _rng(16)
    for (B, H, N, d) in ((1, 1, 1, 1), (1, 2, 7, 3), (2, 3, 33, 8), (1, 2, 130, 64),
                         (1, 1, 257, 128)):
        Q, K, V = _rand_attn(rng, B, H, N, d, std=2.0)
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            O, lse = orc.attn_fwd(Q, K, V, scale, causal)
            Ot, lset = _torch_attn(Q, K, V, scale, causal)
            _close(O, Ot, 1e-12, 1e-12, what=f"sdpa O {B, H, N, d} causal={causal}")
            _close(lse, lset, 1e-12, 1e-12, what=f"logsumexp {B, H, N, d} causal={causal}")


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def pin_softmax_invariants(orc):
    rng = _rng(17)
    x = np.round(rng.standard_normal((6, 301)) * 8.0, 3)
    p = orc.row_softmax(x)
    assert np.all(p > 0.0) and np.all(p <= 1.0), "0 < p <= 1"
    _close(p.sum(axis=1), np.ones(6), 1e-13, what="rows sum to 1")
    _close(orc.row_softmax(x + 37.0), p, 1e-15, 1e-12, what="shift invariance")
    perm = rng.permutation(301)
    _close(orc.row_softmax(x[:, perm]), p[:, perm], 1e-15, 1e-13, what="permutation")


def pin_attn_probabilities(orc):
    # With V = I (N = d) the output row is the probability row itself, which can
    # be brute-forced by the naive softmax (no max subtraction; scores are small).
    rng = _rng(18)
    N = d = 24
    Q = rng.standard_normal((1, 1, N, d))
    K = rng.standard_normal((1, 1, N, d))
    V = np.eye(N).reshape(1, 1, N, d)
    scale = 0.25
    S = scale * (Q[0, 0] @ K[0, 0].T)
    for causal in (False, True):
        O, _ = orc.attn_fwd(Q, K, V, scale, causal)
        P = O[0, 0]
        E = np.exp(S)
        if causal:
            E = np.tril(E)
            assert np.all(P[np.triu_indices(N, 1)] == 0.0), "masked probability must be 0"
        _close(P, E / E.sum(axis=1, keepdims=True), 1e-15, 1e-13,
               what=f"naive softmax causal={causal}")
        _close(P.sum(axis=1), np.ones(N), 1e-14, what="rows of P sum to 1")


def pin_attn_key_shift(orc):
    # Adding u to every key adds scale*q_i.u to every score of row i: P and O
    # are unchanged and lse_i moves by exactly that amount.
    rng = _rng(19)
    B, H, N, d = 1, 2, 40, 8
    Q, K, V = _rand_attn(rng, B, H, N, d)
    u = rng.standard_normal(d)
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        O, lse = orc.attn_fwd(Q, K, V, scale, causal)
        O2, lse2 = orc.attn_fwd(Q, K + u, V, scale, causal)
        _close(O2, O, 1e-12, 1e-12, what="O under key shift")
        _close(lse2, lse + scale * (Q @ u), 1e-12, 1e-12, what="lse under key shift")


def pin_attn_permutations(orc):
    rng = _rng(20)
    B, H, N, d = 1, 1, 31, 5
    Q, K, V = _rand_attn(rng, B, H, N, d)
    O, lse = orc.attn_fwd(Q, K, V, 0.4, False)
    pk = rng.permutation(N)
    O2, lse2 = orc.attn_fwd(Q, K[:, :, pk], V[:, :, pk], 0.4, False)
    _close(O2, O, 1e-13, 1e-13, what="joint key/value permutation")
    _close(lse2, lse, 1e-13, 1e-13, what="lse under key permutation")
    pq = rng.permutation(N)
    O3, lse3 = orc.attn_fwd(Q[:, :, pq], K, V, 0.4, False)
    _close(O3, O[:, :, pq], 0.0, what="query permutation")
    _close(lse3, lse[:, :, pq], 0.0, what="lse under query permutation")


def pin_attn_slices_independent(orc):
    rng = _rng(21)
    B, H, N, d = 2, 3, 17, 4
    Q, K, V = _rand_attn(rng, B, H, N, d)
    for causal in (False, True):
        O, lse = orc.attn_fwd(Q, K, V, 0.6, causal)
        for b in range(B):
            for h in range(H):
                sl = (slice(b, b + 1), slice(h, h + 1))
                O1, lse1 = orc.attn_fwd(Q[sl], K[sl], V[sl], 0.6, causal)
                _close(O[sl], O1, 0.0, what="slice output")
                _close(lse[sl], lse1, 0.0, what="slice lse")


def pin_attn_extreme_scores(orc):
    # Scores of order 1e5: everything stays finite and every output lies in the
    # convex hull of the value rows (each coordinate within [min V, max V]).
    rng = _rng(22)
    B, H, N, d = 1, 1, 50, 8
    Q, K, V = _rand_attn(rng, B, H, N, d)
    for causal in (False, True):
        O, lse = orc.attn_fwd(Q * 1e4, K * 10.0, V, 1.0, causal)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
        lo = V.min(axis=2, keepdims=True) - 1e-12
        hi = V.max(axis=2, keepdims=True) + 1e-12
        assert np.all(O >= lo) and np.all(O <= hi), "output outside the hull of V"


# --------------------------------------------------------------------------
# Brute force: the online recurrence reaches the three-pass result
# --------------------------------------------------------------------------

def pin_online_equals_three_pass(orc):
    rng = _rng(23)
    for N in (1, 2, 3, 5, 8, 17, 33):
        for d in (1, 2, 3, 8):
            Q, K, V = _rand_attn(rng, 1, 2, N, d, std=2.5)
            for causal in (False, True):
                O, lse = orc.attn_fwd(Q, K, V, 0.8, causal)
                for br in sorted({1, 2, 3, 5, N}):
                    for bc in sorted({1, 2, 3, 5, N}):
                        O2, lse2 = orc.attn_online(Q, K, V, 0.8, causal, br, bc)
                        _close(O2, O, 1e-12, 1e-12,
                               what=f"online O N={N} d={d} br={br} bc={bc} c={causal}")
                        _close(lse2, lse, 1e-12, 1e-12,
                               what=f"online lse N={N} d={d} br={br} bc={bc} c={causal}")


def pin_online_trace_final_state(orc):
    # For any block size the final (m, l) of the online trace describes the
    # whole row: m + ln l equals the three-pass lse of the same scores.
    rng = _rng(24)
    for n in (1, 4, 9, 64):
        x = rng.standard_normal(n) * 6.0
        Q, K, V = _scores_as_attention(x, np.zeros(n))
        _, lse = orc.attn_fwd(Q, K, V, 1.0, False)
        for bc in (1, 2, 3, 7, n):
            m, l = orc.online_row_trace(x, bc)
            assert m[-1] == x.max(), "final running max must be the row max"
            _close(m[-1] + math.log(l[-1]), lse[0, 0, 0], 1e-13, 1e-13,
                   what=f"online trace n={n} bc={bc}")


def pin_merge_key_shards(orc):
    # Attention over the union of disjoint key sets, computed whole, equals the
    # merge of the attention over each set (Lesson 22, section 22).  Three
    # shards of N keys each: the whole problem stacks the query block three
    # times so the definition can be evaluated with equal query and key
    # counts; its first N rows are the queries of every shard.
    rng = _rng(31)
    for N, d in ((1, 1), (5, 3), (16, 8)):
        Q, _, _ = _rand_attn(rng, 1, 2, N, d)
        shards = [_rand_attn(rng, 1, 2, N, d, std=1.0 + 2.0 * s)[1:] for s in range(3)]
        Kall = np.concatenate([k for k, _ in shards], axis=2)
        Vall = np.concatenate([v for _, v in shards], axis=2)
        O, lse = orc.attn_fwd(np.concatenate([Q] * 3, axis=2), Kall, Vall, 0.7, False)
        parts = [orc.attn_fwd(Q, k, v, 0.7, False) for k, v in shards]
        Om, lsem = orc.attn_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        _close(Om, O[:, :, :N], 1e-12, 1e-12, what=f"merged O N={N} d={d}")
        _close(lsem, lse[:, :, :N], 1e-12, 1e-12, what=f"merged lse N={N} d={d}")


def pin_merge_causal_halves(orc):
    # Causal attention with the keys cut at c = N / 2.  Keys 0..c-1: rows
    # below c see them causally, rows from c on see all of them; keys c..N-1:
    # rows from c on see them causally (the same problem shifted by c), rows
    # below c see none (lse -inf, output left as NaN: it must not be read).
    rng = _rng(32)
    for N, d in ((2, 1), (8, 4), (32, 8)):
        c = N // 2
        Q, K, V = _rand_attn(rng, 1, 2, N, d, std=1.5)
        O, lse = orc.attn_fwd(Q, K, V, 0.9, True)
        o0 = np.full_like(O, np.nan)
        l0 = np.full_like(lse, np.nan)
        o1 = np.full_like(O, np.nan)
        l1 = np.full_like(lse, -np.inf)
        o0[:, :, :c], l0[:, :, :c] = orc.attn_fwd(Q[:, :, :c], K[:, :, :c], V[:, :, :c], 0.9, True)
        o0[:, :, c:], l0[:, :, c:] = orc.attn_fwd(Q[:, :, c:], K[:, :, :c], V[:, :, :c], 0.9, False)
        o1[:, :, c:], l1[:, :, c:] = orc.attn_fwd(Q[:, :, c:], K[:, :, c:], V[:, :, c:], 0.9, True)
        Om, lsem = orc.attn_merge(np.stack([o0, o1]), np.stack([l0, l1]))
        _close(Om, O, 1e-12, 1e-12, what=f"causal merged O N={N}")
        _close(lsem, lse, 1e-12, 1e-12, what=f"causal merged lse N={N}")


def pin_merge_special_cases(orc):
    # One partial merges to itself; empty partials (-inf) change nothing and
    # their outputs are never read; a row with only empty partials is O = 0,
    # lse = -inf; the order of the partials does not matter.
    rng = _rng(33)
    o = rng.standard_normal((2, 3, 4))
    l = rng.standard_normal((2, 3)) * 5.0
    Om, lsem = orc.attn_merge(o[None], l[None])
    assert np.array_equal(Om, o) and np.array_equal(lsem, l), "single partial must merge to itself"
    empty_o = np.full_like(o, np.nan)
    empty_l = np.full_like(l, -np.inf)
    Om, lsem = orc.attn_merge(np.stack([empty_o, o, empty_o]), np.stack([empty_l, l, empty_l]))
    assert np.array_equal(Om, o) and np.array_equal(lsem, l), "empty partials must change nothing"
    Om, lsem = orc.attn_merge(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(Om == 0.0) and np.all(lsem == -np.inf), "all-empty row must be O = 0, -inf"
    parts_o = rng.standard_normal((5, 2, 3, 4))
    parts_l = rng.standard_normal((5, 2, 3)) * 4.0
    O1, l1 = orc.attn_merge(parts_o, parts_l)
    perm = [3, 0, 4, 2, 1]
    O2, l2 = orc.attn_merge(parts_o[perm], parts_l[perm])
    _close(O2, O1, 1e-13, 1e-13, what="merge order O")
    _close(l2, l1, 1e-13, 1e-13, what="merge order lse")
    # Two equal partials: same output, lse grows by ln 2.
    O3, l3 = orc.attn_merge(np.stack([o, o]), np.stack([l, l]))
    _close(O3, o, 1e-14, 1e-14, what="equal partials O")
    _close(l3, l + math.log(2.0), 1e-14, 1e-14, what="equal partials lse")


def pin_bwd_finite_differences(orc):
    # The gradients of L = sum(dO * O) against central differences of L
    # computed with the forward oracle alone: no gradient formula involved.
    rng = _rng(41)
    h = 1e-6
    for N, d, causal in ((1, 2, False), (3, 2, True), (4, 3, False), (5, 2, True)):
        Q, K, V = _rand_attn(rng, 1, 2, N, d, std=1.2)
        dO = rng.standard_normal(Q.shape)
        grads = orc.attn_bwd(Q, K, V, dO, 0.7, causal)

        def loss(X, which):
            args = [Q, K, V]
            args[which] = X
            O, _ = orc.attn_fwd(*args, 0.7, causal)
            return float((O * dO).sum())

        for which, (X, G) in enumerate(zip((Q, K, V), grads)):
            fd = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += h
                Xm[idx] -= h
                fd[idx] = (loss(Xp, which) - loss(Xm, which)) / (2 * h)
            _close(G, fd, 1e-7, 1e-7, what=f"grad {'QKV'[which]} N={N} d={d} causal={causal}")


def pin_bwd_library(orc):
    # torch autograd in float64 through a plain softmax attention.
    import torch
    rng = _rng(42)
    for causal in (False, True):
        Q, K, V = _rand_attn(rng, 2, 3, 17, 8)
        dO = rng.standard_normal(Q.shape)
        q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
        s = 0.35 * (q @ k.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(17, 17, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ v
        o.backward(torch.tensor(dO))
        got = orc.attn_bwd(Q, K, V, dO, 0.35, causal)
        for name, g, t in zip("QKV", got, (q, k, v)):
            _close(g, t.grad.numpy(), 1e-12, 1e-10, what=f"torch grad {name} causal={causal}")


def pin_bwd_invariants(orc):
    # Adding one vector to every key leaves each softmax row unchanged, so the
    # key gradients sum to zero; the probabilities of a row sum to one, so the
    # value gradients sum to the sum of dO.  One key: P = 1 whatever Q and K,
    # so dQ = dK = 0 and dV = dO.  dO = 0 gives zero gradients.
    rng = _rng(43)
    for causal in (False, True):
        Q, K, V = _rand_attn(rng, 1, 2, 9, 4, std=1.5)
        dO = rng.standard_normal(Q.shape)
        dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, 0.6, causal)
        _close(dK.sum(axis=2), np.zeros((1, 2, 4)), 1e-12, what=f"sum dK causal={causal}")
        _close(dV.sum(axis=2), dO.sum(axis=2), 1e-12, 1e-12, what=f"sum dV causal={causal}")
        z = orc.attn_bwd(Q, K, V, np.zeros_like(dO), 0.6, causal)
        assert all(np.all(g == 0.0) for g in z), "dO = 0 must give zero gradients"
    Q, K, V = _rand_attn(rng, 2, 1, 1, 5)
    dO = rng.standard_normal(Q.shape)
    dQ, dK, dV = orc.attn_bwd(Q, K, V, dO, 0.9, False)
    assert np.all(dQ == 0.0) and np.all(dK == 0.0), "one key: dQ = dK = 0"
    assert np.array_equal(dV, dO), "one key: dV = dO"


# --------------------------------------------------------------- FP8 inputs --
def pin_fp8_decode_values(orc):
    # The E4M3 encoding written out: zero and negative zero, the smallest and
    # largest subnormals (2^-9, 7 * 2^-9), the smallest normal 2^-6, 1, 1.5, 2,
    # the largest finite 448 and its negative, the two NaN codes; and the
    # scale multiplies.
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x7E, 0xFE, 0x7F, 0xFF],
                     dtype=np.uint8)
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 2.0, 448.0, -448.0]
    got = orc.fp8_decode(codes)
    assert list(got[:10]) == want, got
    assert np.signbit(got[1]) and np.isnan(got[10]) and np.isnan(got[11])
    np.testing.assert_array_equal(orc.fp8_decode(codes[:10], 0.25), np.array(want) * 0.25)


def pin_fp8_decode_library(orc):
    # Every one of the 256 codes against torch's float8_e4m3fn conversion, an
    # independent implementation of the same encoding.
    import torch
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.fp8_decode(codes)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], lib[~nan])


def _e4m3_grid():
    """All finite E4M3 values (code, value), from the decode pins' encoding."""
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    return codes


def pin_fp8_encode_grid(orc):
    # Every finite code encodes back to itself; a midpoint between two
    # neighbouring codes goes to the one with the even mantissa field (the even
    # code), and a value a hair off the midpoint to the nearer code; the scale
    # divides; values past 448 have no code.
    codes = _e4m3_grid()
    vals = orc.fp8_decode(codes)
    np.testing.assert_array_equal(orc.fp8_encode(vals), codes)
    pos = np.arange(0x00, 0x7E, dtype=np.uint8)  # each with its upper neighbour
    lo, hi = orc.fp8_decode(pos), orc.fp8_decode(pos + 1)
    mid = 0.5 * (lo + hi)
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    np.testing.assert_array_equal(orc.fp8_encode(mid), even)
    np.testing.assert_array_equal(orc.fp8_encode(-mid), even | 0x80)
    np.testing.assert_array_equal(orc.fp8_encode(np.nextafter(mid, 0)), pos)
    np.testing.assert_array_equal(orc.fp8_encode(np.nextafter(mid, 1e9)), (pos + 1).astype(np.uint8))
    np.testing.assert_array_equal(orc.fp8_encode(vals * 0.375, 0.375), codes)
    for bad in (448.5, np.nan, -np.inf):
        try:
            orc.fp8_encode(np.array([bad]))
        except RuntimeError:
            continue
        raise AssertionError(f"{bad} was encoded")


def pin_fp8_encode_library(orc):
    # Against torch's float8_e4m3fn conversion (round to nearest even, an
    # independent implementation) on float32 values spread over the whole
    # finite range, subnormals and signed zeros included.
    import torch
    rng = _rng(70)
    x = (rng.uniform(-1, 1, 20000) * np.exp2(rng.integers(-14, 9, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.fp8_encode(x.astype(np.float64)), lib)


def pin_hadamard_library(orc):
    # With all signs +1 the rotation of the identity is H / sqrt(d), H from
    # scipy's Sylvester construction; a sign flips its input column.
    import scipy.linalg
    for d in (1, 2, 4, 32, 128):
        H = scipy.linalg.hadamard(d).astype(np.float64)
        _close(orc.hadamard_rotate(np.eye(d), np.ones(d)), H / np.sqrt(d), 1e-15,
               what=f"H_{d}")
    rng = _rng(71)
    X = rng.standard_normal((5, 64))
    s = rng.choice([-1.0, 1.0], 64)
    _close(orc.hadamard_rotate(X, s), orc.hadamard_rotate(X * s, np.ones(64)), 1e-14,
           what="signs act on input columns")


def pin_hadamard_orthogonal(orc):
    # M M^T = I, so (Q M)(K M)^T = Q K^T and norms are kept; H is its own
    # inverse up to d, so rotating twice with unit signs returns the input.
    rng = _rng(72)
    Q, K = rng.standard_normal((20, 128)), rng.standard_normal((30, 128))
    s = rng.choice([-1.0, 1.0], 128)
    Qr, Kr = orc.hadamard_rotate(Q, s), orc.hadamard_rotate(K, s)
    _close(Qr @ Kr.T, Q @ K.T, 1e-12, what="scores")
    _close(np.linalg.norm(Qr, axis=1), np.linalg.norm(Q, axis=1), 1e-12, what="norms")
    one = np.ones(128)
    _close(orc.hadamard_rotate(orc.hadamard_rotate(Q, one), one), Q, 1e-12, what="H H = d I")


def pin_mx_rows_definition(orc):
    # Per block of 32: the scale is the smallest power of two 2^e with
    # amax <= 448 * 2^e (byte e + 127; e = 0 for a zero block), hand-checked
    # on edge blocks, and each element decodes to the nearest point of the
    # scaled E4M3 grid (brute force over every code).
    Y = np.zeros((6, 64))
    Y[0, :32] = 1.0
    Y[0, 0] = 448.0              # amax exactly 448 -> e = 0
    Y[1, 0] = 449.0              # just above -> e = 1
    Y[2, :32] = -224.0           # 224 = 448 / 2 -> e = -1
    Y[3, 32:] = 0.75 * 2.0 ** -20  # tiny block
    rng = _rng(73)
    Y[4] = rng.standard_normal(64) * 3
    Y[5] = rng.standard_normal(64) * np.exp2(rng.integers(-6, 6, 64))
    codes, sc = orc.mx_quantize_rows(Y)
    assert sc.shape == (6, 2)
    assert list(sc[:4, 0]) == [127, 128, 126, 127] and sc[3, 1] == 127 + (-29), sc
    e = sc.astype(np.int64) - 127
    amax = np.abs(Y).reshape(6, 2, 32).max(axis=2)
    nz = amax > 0
    assert np.all(amax <= 448.0 * np.exp2(e)) and np.all(amax[nz] > 224.0 * np.exp2(e[nz]))
    grid_codes = _e4m3_grid()
    grid = orc.fp8_decode(grid_codes)
    dec = orc.mx_decode_rows(codes, sc)
    for r in range(6):
        for t in range(64):
            g = grid * np.exp2(e[r, t // 32])
            dist = np.abs(g - Y[r, t])
            best = dist.min()
            assert abs(dec[r, t] - Y[r, t]) == best, (r, t, dec[r, t], Y[r, t])


def pin_mx_cols_transpose(orc):
    # Column blocks are row blocks of the transposed slice: quantizing the
    # rows of each column of V in blocks of 32 equals quantizing the rows of
    # V^T; a ragged last block (n = 45) behaves as if padded with zeros.
    rng = _rng(74)
    V = rng.standard_normal((2, 3, 64, 32)) * np.exp2(rng.integers(-4, 4, (2, 3, 64, 32)))
    c, s = orc.mx_quantize_cols(V)
    cr, sr = orc.mx_quantize_rows(np.swapaxes(V, -1, -2))
    np.testing.assert_array_equal(c, np.swapaxes(cr, -1, -2))
    np.testing.assert_array_equal(s, np.swapaxes(sr, -1, -2))
    W = V[:, :, :45]
    cw, sw = orc.mx_quantize_cols(W)
    Wp = np.concatenate([W, np.zeros((2, 3, 19, 32))], axis=2)
    cp, sp = orc.mx_quantize_cols(Wp)
    np.testing.assert_array_equal(cw, cp[:, :, :45])
    np.testing.assert_array_equal(sw, sp)
    _close(orc.mx_decode_cols(cw, sw), orc.mx_decode_cols(cp, sp)[:, :, :45], 0.0)


def pin_mx_decode_values(orc):
    # value(code) * 2^(byte - 127): 1.0 at byte 130 is 8, -2 at byte 120 is
    # -2^-6, the largest subnormal at byte 127 is 7 * 2^-9.
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :3] = [0x38, 0xC0, 0x07]
    for byte, want in ((130, [8.0, -16.0, 7 * 2.0 ** -6]), (120, [2.0 ** -7, -(2.0 ** -6), 7 * 2.0 ** -16])):
        got = orc.mx_decode_rows(codes, np.array([[byte]], dtype=np.uint8))
        assert list(got[0, :3]) == want and not got[0, 3:].any(), (byte, got[0, :3])
    cv = np.zeros((33, 1), dtype=np.uint8)
    cv[0, 0], cv[32, 0] = 0x38, 0x38
    got = orc.mx_decode_cols(cv, np.array([[127], [129]], dtype=np.uint8))
    assert got[0, 0] == 1.0 and got[32, 0] == 4.0


def pin_attn_fp8_mx_unit_scales(orc):
    # With every block scale 2^0 the block-quantized attention is the FP8
    # attention with unit tensor scales.
    rng = _rng(75)
    B, H, N, d = 1, 2, 40, 64
    Q8, K8, V8 = (rng.integers(0, 256, (B, H, N, d)).astype(np.uint8) & 0xB7 for _ in range(3))
    one_r = np.full((B, H, N, d // 32), 127, dtype=np.uint8)
    one_c = np.full((B, H, (N + 31) // 32, d), 127, dtype=np.uint8)
    for causal in (False, True):
        a = orc.attn_fwd_fp8_mx(Q8, one_r, K8, one_r, V8, one_c, 0.125, causal)
        b = orc.attn_fwd_fp8(Q8, K8, V8, 1.0, 1.0, 1.0, 0.125, causal)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def pin_incoherent_processing_outliers(orc):
    # The claim of the FP8 section: with outliers, one scale per tensor loses
    # accuracy that block scales after a random-sign Hadamard rotation of Q
    # and K recover (the pages report a 2.6x lower RMSE of O).  Inputs: N(0,1)
    # with four head channels of Q and K scaled by 20; O compared with exact
    # attention on the unquantized values.
    rng = _rng(76)
    B, H, N, d = 1, 2, 256, 128
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    ch = rng.choice(d, 4, replace=False)
    Q[..., ch] *= 20.0
    K[..., ch] *= 20.0
    scale = 1.0 / np.sqrt(d)
    O, _ = orc.attn_fwd(Q, K, V, scale, False)

    def tensor_q(X):
        s = np.nextafter(np.abs(X).max() / 448.0, np.inf)
        return orc.fp8_decode(orc.fp8_encode(X, s), s)

    def rows_q(X):
        return orc.mx_decode_rows(*orc.mx_quantize_rows(X))

    Vb = orc.mx_decode_cols(*orc.mx_quantize_cols(V))
    Ot, _ = orc.attn_fwd(tensor_q(Q), tensor_q(K), tensor_q(V), scale, False)
    s = rng.choice([-1.0, 1.0], d)
    Or, _ = orc.attn_fwd(rows_q(orc.hadamard_rotate(Q, s)), rows_q(orc.hadamard_rotate(K, s)),
                         Vb, scale, False)
    rmse_t = np.sqrt(np.mean((Ot - O) ** 2))
    rmse_r = np.sqrt(np.mean((Or - O) ** 2))
    assert rmse_r * 2.0 < rmse_t, (rmse_t, rmse_r)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
