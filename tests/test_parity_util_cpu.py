"""Host logic of the parity helpers (no GPU): the gate evaluation names every
gate a statistics record fails, and the relative Frobenius distance of two
Hessians reads only their lower triangles."""

import numpy as np
import pytest

from parity_util import CODE_FRAC, H_TOL, LOSS_TOL, assert_gates, failed_gates, lower_rel_fro


def _passing():
    return {"h_rel": 1e-8, "lam_rel": 1e-9, "u_lower_zero": True, "u_rel": 1e-5, "u_bound": 1e-2, "hard": 0,
            "zero_hard": 0, "identical": 0.99999, "loss_rel": 1e-5, "row_loss_rel_follow": 1e-3,
            "row_loss_rel_free": 1e-3, "loss_gpu": 1.0, "loss_rtn": 2.0, "w_hat_exact": True, "pack_exact": True,
            "scale_rel": 1e-5, "scale_tol": 1.4e-4, "obs_rel": 1e-4}


# each gate with a value just past its threshold
_BREAKS = [("h_rel", 2 * H_TOL), ("lam_rel", 2e-6), ("u_lower_zero", False), ("u_rel", 2e-2), ("hard", 1),
           ("zero_hard", 1), ("identical", CODE_FRAC - 1e-6), ("loss_rel", 2 * LOSS_TOL),
           ("row_loss_rel_follow", 2 * LOSS_TOL), ("row_loss_rel_free", 2 * LOSS_TOL), ("w_hat_exact", False),
           ("pack_exact", False), ("scale_rel", 2e-4), ("obs_rel", 2 * LOSS_TOL)]


def test_a_passing_record_has_no_failed_gate():
    assert failed_gates(_passing()) == []
    assert_gates(_passing())


@pytest.mark.parametrize("key,value", _BREAKS, ids=[k for k, _ in _BREAKS])
def test_each_gate_is_named_when_it_fails(key, value):
    stats = _passing()
    stats[key] = value
    assert failed_gates(stats) == [key]
    with pytest.raises(AssertionError, match=key):
        assert_gates(stats)


def test_loss_at_or_above_rtn_fails():
    stats = _passing()
    stats["loss_gpu"] = stats["loss_rtn"]
    assert failed_gates(stats) == ["loss_below_rtn"]


def test_lower_rel_fro_ignores_the_upper_triangle():
    rng = np.random.default_rng(3)
    d = 300
    b = rng.standard_normal((d, d))
    b = b + b.T
    a = b + 1e-6 * rng.standard_normal((d, d))
    a = np.tril(a)
    a[np.triu_indices(d, 1)] = np.nan  # never written by the library
    full = lambda m: np.tril(m) + np.tril(m, -1).T
    want = np.linalg.norm(full(np.nan_to_num(a)) - b) / np.linalg.norm(b)
    for rows in (64, 128, 2048):
        got = lower_rel_fro(a, b, rows=rows)
        assert np.isfinite(got)
        assert abs(got - want) <= 1e-12 * want
