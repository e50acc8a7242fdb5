"""Pins of the oracle's act-order (desc_act) and static-group path.

The pages name the two options only ([ZLY] "实践指南" / "超参数选择" pass and
list desc_act; [CSDN]'s parameter table lists --desc_act and --static_groups).
The oracle reads them as: quantize the columns in descending H_jj (ties in
index order); without static groups the groups are runs of g columns in that
order, fitted on the current weights; with static groups each column keeps the
grid of its natural group, fitted on the original weights before the loop.

These tests check that reading through facts that do not re-type it: brute
force on the order, exact reductions to round-to-nearest when nothing
propagates, the identity order, and the least-squares re-solve in natural
coordinates at every step.
"""

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(777)


def _sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_act_order_perm_brute_force_with_ties():
    """Selection sort in pure Python: repeatedly take the largest remaining
    diagonal entry, the lowest index among equal ones."""
    diag = [3.0, 5.0, 5.0, 0.0, 7.5, 3.0, 5.0, 1e-300, 0.0]
    h = np.diag(diag) + np.triu(np.ones((9, 9)), 1) * 0.125  # off-diagonal entries do not matter
    left = list(range(len(diag)))
    want = []
    while left:
        best = left[0]
        for c in left[1:]:
            if diag[c] > diag[best]:
                best = c
        want.append(best)
        left.remove(best)
    assert O.act_order_perm(h).tolist() == want == [4, 1, 2, 6, 0, 5, 7, 3, 8]


def _diagonal_h_layer(m, d, n=128):
    """Hadamard token columns scaled per column by distinct powers of two and
    small odd integers: H = 2n diag(a^2), exactly, in a shuffled order."""
    a = np.array([(1 + 2 * (k % 5)) * 2.0 ** -(k % 7) for k in range(d)])
    a = a[RNG.permutation(d)]
    x = (_sylvester(n)[:, :d] * a).astype(np.float16)
    assert np.all(x.astype(np.float64) == _sylvester(n)[:, :d] * a)
    w = RNG.standard_normal((m, d)) * 0.02
    return w, x


@pytest.mark.parametrize("group,grid,bits", [(8, "asym", 3), (16, "ternary", 2), (4, "asym", 4)])
def test_diagonal_h_act_order_is_rtn_over_permuted_groups(group, grid, bits):
    """H diagonal: U is diagonal and nothing propagates, so act-order without
    static groups is round-to-nearest with group k = the columns
    perm[k g : (k+1) g], fitted on the original weights of exactly those
    columns."""
    m, d = 12, 32
    w, x = _diagonal_h_layer(m, d)
    res, g_idx, perm, h, u, _ = O.quantize_layer_act_order(w, x, bits, grid, group, block=8)
    np.testing.assert_array_equal(np.triu(u, 1), 0)
    assert np.all(np.diff(np.diag(h)[perm]) <= 0)
    for k in range(d // group):
        cols = perm[k * group:(k + 1) * group]
        rtn = O.rtn_quantize(w[:, cols], bits, grid, 0)  # one grid over the gathered columns
        np.testing.assert_array_equal(res.codes[:, cols], rtn.codes)
        np.testing.assert_allclose(res.w_hat[:, cols], rtn.w_hat, rtol=1e-15)
        np.testing.assert_array_equal(res.scales[:, k], rtn.scales[:, 0])
        np.testing.assert_array_equal(res.zeros[:, k], rtn.zeros[:, 0])
        assert np.all(g_idx[cols] == k)


@pytest.mark.parametrize("group,grid,bits", [(8, "asym", 3), (16, "ternary", 2)])
def test_diagonal_h_static_groups_is_rtn_over_natural_groups(group, grid, bits):
    """H diagonal with static groups: exactly round-to-nearest per natural group."""
    m, d = 10, 32
    w, x = _diagonal_h_layer(m, d)
    res, g_idx, perm, _, _, _ = O.quantize_layer_act_order(w, x, bits, grid, group, static_groups=True, block=8)
    assert perm.tolist() != list(range(d))
    rtn = O.rtn_quantize(w, bits, grid, group)
    np.testing.assert_array_equal(res.codes, rtn.codes)
    np.testing.assert_allclose(res.w_hat, rtn.w_hat, rtol=1e-15)
    np.testing.assert_array_equal(res.scales, rtn.scales)
    np.testing.assert_array_equal(res.zeros, rtn.zeros)
    np.testing.assert_array_equal(g_idx, np.arange(d) // group)


def test_diagonal_h_per_row_grid_is_rtn():
    m, d = 9, 32
    w, x = _diagonal_h_layer(m, d)
    for static in (False, True):
        res, g_idx, _, _, _, _ = O.quantize_layer_act_order(w, x, 4, "asym", 0, static_groups=static, block=8)
        rtn = O.rtn_quantize(w, 4, "asym", 0)
        np.testing.assert_array_equal(res.codes, rtn.codes)
        np.testing.assert_array_equal(g_idx, 0)


def test_identity_order_equals_natural_order():
    """Columns scaled so that diag(H) strictly decreases in natural order: the
    order is the identity and the result is the natural-order one, bit for
    bit (the same arithmetic in the same order)."""
    m, d, n = 16, 48, 400
    mix = RNG.standard_normal((d, d)) * 0.3 + np.eye(d)
    x = RNG.standard_normal((n, d)) @ mix
    x = x / np.linalg.norm(x, axis=0) * np.linspace(40.0, 4.0, d)
    x = x.astype(np.float16)
    w = RNG.standard_normal((m, d)) * 0.02
    res_a, g_idx, perm, _, _, _ = O.quantize_layer_act_order(w, x, 3, "asym", 16, block=8)
    assert perm.tolist() == list(range(d))
    res_n, _, _, _ = O.quantize_layer(w, x, 3, "asym", 16, block=8)
    np.testing.assert_array_equal(res_a.codes, res_n.codes)
    np.testing.assert_array_equal(res_a.w_hat, res_n.w_hat)
    np.testing.assert_array_equal(res_a.scales, res_n.scales)
    np.testing.assert_array_equal(g_idx, np.arange(d) // 16)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("group,static", [(0, False), (4, False), (4, True)])
def test_least_squares_resolve_in_natural_coordinates(seed, group, static):
    """At every step, with the columns already quantized (the set P, in the
    act-order) fixed at their values q, the weight the loop rounds equals the
    least-squares re-solve of the remaining columns F in NATURAL coordinates,
    w~_F = w_F + H_FF^-1 H_FP (w_P - q_P), with the unpermuted damped H. A wrong
    permutation of H, of W or of the outputs fails it."""
    rng = np.random.default_rng(seed)
    m, d, n = 3, 8, 80
    x = (rng.standard_normal((n, d)) @ (rng.standard_normal((d, d)) * 0.5 + np.eye(d))
         * rng.uniform(0.3, 3.0, d)).astype(np.float16)
    w = rng.standard_normal((m, d)) * 0.2
    res, g_idx, perm, h, u, lam = O.quantize_layer_act_order(w, x, 2, "asym", group, static_groups=static,
                                                             block=4)
    assert perm.tolist() != list(range(d))
    hd = h + lam * np.eye(d)
    for j in range(d):
        c = perm[j]
        done, rest = perm[:j], perm[j:]
        w_tilde = w[:, rest].copy()
        if j:
            corr = np.linalg.solve(hd[np.ix_(rest, rest)], hd[np.ix_(rest, done)] @ (w[:, done] - res.w_hat[:, done]).T)
            w_tilde += corr.T
        gi = g_idx[c]
        got = (res.p[:, c] - res.zeros[:, gi]) * res.scales[:, gi]
        np.testing.assert_allclose(got, w_tilde[:, 0], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(res.w_hat[:, c], res.scales[:, gi] * (res.codes[:, c] - res.zeros[:, gi]),
                                   rtol=1e-15)
    if static:
        s_nat, z_nat = O.static_group_grids(w, 2, "asym", group)
        np.testing.assert_array_equal(res.scales, s_nat)
        np.testing.assert_array_equal(res.zeros, z_nat)


def test_follow_mode_maps_positions_to_natural_columns():
    """A planted wrong code (far from any boundary) at a natural column is
    reported as a hard mismatch at that natural column."""
    m, d, n = 4, 16, 100
    x = (RNG.standard_normal((n, d)) * RNG.uniform(0.5, 2.0, d)).astype(np.float16)
    w = RNG.standard_normal((m, d)) * 0.05
    res, _, perm, _, _, _ = O.quantize_layer_act_order(w, x, 4, "asym", 0, block=4)
    planted = res.codes.copy()
    col = int(perm[5])
    far = np.argmax(res.dist[:, col])
    planted[far, col] = (planted[far, col] + 3) % 16
    res2, _, _, _, _, _ = O.quantize_layer_act_order(w, x, 4, "asym", 0, block=4, follow_codes=planted)
    assert res2.hard_mismatch >= 1
    assert (int(far), col) in res2.hard_positions


def test_static_zero_follow_mode_at_an_exact_tie():
    """A group whose extremes are -a and +a has -lo/s = maxq/2 exactly, a
    half-integer: either neighbour is a legitimate zero point in finite
    precision. Follow mode takes the other neighbour as a band mismatch; a
    zero two steps away is a hard mismatch."""
    m, d, g = 2, 8, 4
    w = np.array([[-0.5, 0.25, 0.5, 0.125, 0.3, -0.2, 0.1, 0.05],
                  [0.1, 0.2, 0.3, 0.4, -0.1, -0.2, -0.3, 0.05]])
    s_g, z_g = O.static_group_grids(w, 4, "asym", g)
    assert -(-0.5) / s_g[0, 0] == pytest.approx(7.5, abs=1e-12)
    u = np.eye(d)
    perm = np.arange(d)[::-1].copy()
    other = z_g.copy()
    other[0, 0] = 15 - z_g[0, 0]  # the other side of 7.5
    res, _ = O.gptq_quantize_ordered(w, u, perm, 4, "asym", g, True, follow_zeros=other)
    assert (res.zero_band_mismatch, res.zero_hard_mismatch) == (1, 0)
    assert res.zeros[0, 0] == other[0, 0]
    far = z_g.copy()
    far[1, 1] += 2
    res2, _ = O.gptq_quantize_ordered(w, u, perm, 4, "asym", g, True, follow_zeros=far)
    assert res2.zero_hard_mismatch == 1
