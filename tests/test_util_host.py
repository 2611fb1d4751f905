"""The parity helpers themselves: a NaN or a wrong infinity in a GPU result
must fail every comparison (CPU only)."""
import numpy as np
import pytest

from _util import assert_close, max_err


def _case():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((2, 3, 5, 8))
    lse = rng.standard_normal((2, 3, 5))
    lse[0, 0, 0] = -np.inf  # a row with no visible key
    o[0, 0, 0] = 0.0
    return o, lse


def test_identical_results_pass():
    o, lse = _case()
    assert assert_close(o.copy(), lse.copy(), o, lse, "f32") == (0.0, 0.0)


@pytest.mark.parametrize("where", ["o", "lse"])
def test_nan_fails_assert_close(where):
    o, lse = _case()
    go, gl = o.copy(), lse.copy()
    if where == "o":
        go[1, 2, 3, 4] = np.nan
    else:
        gl[1, 2, 3] = np.nan
    with pytest.raises(AssertionError):
        assert_close(go, gl, o, lse, "bf16")


def test_nan_in_the_masked_row_fails():
    o, lse = _case()
    gl = lse.copy()
    gl[0, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        assert_close(o.copy(), gl, o, lse, "bf16")


@pytest.mark.parametrize("bad", [-np.inf, np.inf])
def test_infinite_lse_where_oracle_is_finite_fails(bad):
    o, lse = _case()
    gl = lse.copy()
    gl[1, 1, 1] = bad
    with pytest.raises(AssertionError):
        assert_close(o.copy(), gl, o, lse, "bf16")


def test_finite_lse_where_oracle_is_neg_inf_fails():
    o, lse = _case()
    gl = lse.copy()
    gl[0, 0, 0] = -80.0
    with pytest.raises(AssertionError):
        assert_close(o.copy(), gl, o, lse, "bf16")


def test_max_err_nan_and_inf():
    assert max_err([np.nan, 1.0], [1.0, 1.0]) == np.inf
    assert max_err([np.inf, 1.0], [1.0, 1.0]) == np.inf
    assert max_err([-np.inf, 1.0], [np.inf, 1.0]) == np.inf
    assert max_err([-np.inf, 1.5], [-np.inf, 1.0]) == 0.5
    assert max_err([], []) == 0.0


def test_max_err_rejects_unevaluated_oracle_entries():
    with pytest.raises(ValueError):
        max_err([1.0, 1.0], [np.nan, 1.0])


def test_max_err_shape_mismatch():
    with pytest.raises(AssertionError):
        max_err(np.zeros(3), np.zeros(4))
