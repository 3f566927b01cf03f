"""Per-element error contract of the fp8 attention forward (attn_fwd_fp8 and
attn_fwd_fp8_mx) against exact attention on the values its inputs stand for.

The reference is exact attention on the values the fp8 codes stand for
(oracle.attn_fwd_fp8 or oracle.attn_fwd_fp8_mx: the oracle's own E4M3 and
block-scale decoding, then oracle.attn_fwd).
The kernel adds three roundings, each modelled from its definition or a
measurement:
  * the scores: the matrix cores form the fp8 products exactly but sum each
    64-term block at reduced precision.  On this GPU the error of a 128-term
    dot product measured at most 2.7e-5 of its sum of |products| on Gaussian
    data stored as E4M3 (test_gpu_fp8.test_fp8_score_sum_error), 1e-4 on codes drawn
    at random from the whole range; the bar takes EPS_S = 2^-13 of that sum:
        dS_ij = EPS_S * scale * sum_d |Q_id K_jd|;
    lse_i then moves by at most max_j dS_ij, O_it by at most
    sum_j P_ij dS_ij |V_jt - O_it| <= sum_j P_ij dS_ij (|V_jt| + |O_it|);
  * each probability rounded to fp8 before the P V product: E4M3 keeps 3
    mantissa bits, so a normal value x rounds to nearest with an error up to
    u8 x (u8 = 2^-4), of standard deviation u8 x / sqrt(3) for uniformly
    placed x.  The kernel forms p' = 16 P / P_max or larger (its reference
    trails the row maximum), so a probability below 2^-10 P_max may be
    subnormal in fp8 and err by up to 2^-10 in p' units, at most 2^-14 P_max
    in P.  Independent, zero-mean roundings give element (i, t) of O the
    standard deviation
        sigma_it = sqrt( sum_j (u8 P_ij V_jt)^2 / 3
                         + sum_{j: P_ij < 2^-10 P_i,max} (2^-14 P_i,max V_jt)^2 / 3 );
  * O rounded to bf16: 2^-8 |O_it|.
The bars: |err O_it| <= 6 sigma_it + sum_j P_ij dS_ij (|V_jt| + |O_it|)
+ 2^-8 |O_it| + 1e-4, and |err lse_i| <= max_j dS_ij + 1e-4.
"""
from __future__ import annotations

import numpy as np

U8 = 2.0 ** -4      # unit roundoff of E4M3 (3 mantissa bits)
EPS_S = 2.0 ** -13  # score error per sum of |products| (fp8 matrix-core sums)
ELEM_FACTOR = 6.0


def _bars(Qd, Kd, Vd, scale, causal):
    """Per-element bars of O and per-row bars of lse for one (b, h) slice (the
    module docstring), from its decoded inputs in fp64."""
    S = scale * (Qd @ Kd.T)
    dS = EPS_S * scale * (np.abs(Qd) @ np.abs(Kd).T)
    N = S.shape[0]
    if causal:
        hidden = np.triu(np.ones((N, N), dtype=bool), 1)
        S[hidden] = -np.inf
        dS[hidden] = 0.0
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    O = P @ Vd
    pmax = P.max(axis=1, keepdims=True)
    sub = ((P < 2.0 ** -10 * pmax) * (2.0 ** -14 * pmax)) ** 2
    sigma = np.sqrt(((U8 * P) ** 2 @ Vd ** 2 + sub @ Vd ** 2) / 3.0)
    PdS = P * dS
    score_term = PdS @ np.abs(Vd) + PdS.sum(axis=1, keepdims=True) * np.abs(O)
    o_bar = ELEM_FACTOR * sigma + score_term + 2.0 ** -8 * np.abs(O) + 1e-4
    lse_bar = dS.max(axis=1) + 1e-4
    return o_bar, lse_bar
