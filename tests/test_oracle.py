"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rows_sampler_matches_full(orc):
    # The sampled-row entry point evaluates the same per-row definition.
    rng = np.random.default_rng(5)
    Q, K, V = (rng.standard_normal((2, 3, 45, 16)) for _ in range(3))
    for causal in (False, True):
        O, lse = orc.attn_fwd(Q, K, V, 0.25, causal)
        bh = np.array([0, 5, 3, 2, 4])
        qi = np.array([0, 44, 17, 3, 30])
        Or, lser = orc.attn_rows(Q, K, V, 0.25, causal, bh, qi)
        np.testing.assert_array_equal(Or, O.reshape(6, 45, 16)[bh, qi])
        np.testing.assert_array_equal(lser, lse.reshape(6, 45)[bh, qi])


def test_bad_arguments_are_rejected(orc):
    with pytest.raises(RuntimeError):
        orc.attn_rows(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)),
                      np.zeros((1, 1, 4, 2)), 1.0, False, [1], [0])
    with pytest.raises(RuntimeError):
        orc.online_row_trace(np.zeros(3), 0)


def test_empty_inputs(orc):
    O, lse = orc.attn_fwd(np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 4)),
                          np.zeros((1, 2, 0, 4)), 1.0, True)
    assert O.shape == (1, 2, 0, 4) and lse.shape == (1, 2, 0)
    assert orc.row_softmax(np.zeros((0, 5))).shape == (0, 5)
