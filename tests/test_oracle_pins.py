"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
from fractions import Fraction

import pytest

import oracle
import pins


def test_three_option_example_in_exact_fractions():
    """The page's worked example, recomputed in exact fractions."""
    g, got = pins.three_option_fractions()
    for key, val in got.items():
        assert val == [Fraction(x) for x in g[key]], key
    assert got["naive_output"] != got["output"]


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_pin(name):
    errs = pins.ALL_PINS[name](oracle.default())
    assert not errs, "\n".join(errs[:10])


def test_oracle_rejects_malformed_arguments():
    import numpy as np
    t = np.zeros((1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.verify(t, None, np.zeros((1, 1), np.int32), temperature=0.0)  # T must be > 0
    with pytest.raises(ValueError):
        oracle.verify(t, np.zeros((1, 1, 4), np.float32), np.zeros((1, 1), np.int32),
                      np.array([3], np.int32), temperature=1.0)  # gamma_i > gamma_max


def test_flags_for_bad_tokens_and_nonfinite_rows():
    import numpy as np
    t = np.zeros((2, 2, 4), np.float32)
    t[1, 0, 2] = np.nan
    q = np.zeros((2, 1, 4), np.float32)
    d = np.array([[7], [0]], np.int32)
    r = oracle.verify(t, q, d, temperature=1.0, seed=3)
    assert r["flags"][0] & oracle.FLAG_TOKEN_RANGE and r["accept_count"][0] == 0
    assert r["flags"][1] & oracle.FLAG_NONFINITE
