"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the fact it checks. None of them re-types the oracle's
formula: they use closed forms, exact special cases, brute force on tiny
inputs, library routines used in another way, and invariants, chosen so that a
dropped term, a wrong sign or index, or a transposed operand fails one of them.
"""

import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(20240)


# ---------------------------------------------------------------------------
# H = 2 X^T X
# ---------------------------------------------------------------------------
def test_hessian_brute_force_tiny():
    """Pure-Python triple loop in exact rationals on a 5-token x 3-feature X."""
    x = np.array([[1, -2, 0.5], [3, 0.25, -1], [0, 1, 1], [-1.5, 2, 4], [2, 2, -2]])
    h = O.hessian(x)
    for i in range(3):
        for j in range(3):
            exact = 2 * sum(Fraction(x[t, i]) * Fraction(x[t, j]) for t in range(5))
            assert h[i, j] == float(exact)


def test_hessian_one_hot_tokens_is_diagonal_counts():
    """Token t = e_(t mod d): H = 2 diag(counts) exactly."""
    d, n = 7, 30
    x = np.zeros((n, d), np.float16)
    for t in range(n):
        x[t, t % d] = 1
    counts = np.bincount(np.arange(n) % d, minlength=d)
    np.testing.assert_array_equal(O.hessian(x), 2.0 * np.diag(counts))


def _sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_hessian_hadamard_columns_give_scaled_identity():
    """d columns of a +-1 Sylvester Hadamard matrix of order N: H = 2N I."""
    n, d = 64, 24
    x = _sylvester(n)[:, :d].astype(np.float16)
    np.testing.assert_array_equal(O.hessian(x), 2.0 * n * np.eye(d))


def test_hessian_chunking_is_a_sum():
    x = RNG.standard_normal((300, 9)).astype(np.float16)
    whole = O.hessian(x)
    parts = O.hessian([x[:100], x[100:257], x[257:]])
    np.testing.assert_allclose(parts, whole, rtol=1e-14, atol=1e-12)


# ---------------------------------------------------------------------------
# damping
# ---------------------------------------------------------------------------
def test_damp_hand_value():
    h = np.array([[2.0, 1.0, 0.0], [1.0, 4.0, 1.0], [0.0, 1.0, 6.0]])
    hd, lam = O.damp(h, 0.01)
    assert lam == pytest.approx(0.04)           # 1 % of mean(2, 4, 6) = 4
    np.testing.assert_allclose(np.diag(hd), [2.04, 4.04, 6.04], rtol=1e-15)
    assert hd[0, 1] == 1.0 and hd[2, 0] == 0.0  # off-diagonal untouched


# ---------------------------------------------------------------------------
# U = chol(H_d^-1), upper
# ---------------------------------------------------------------------------
def test_u_two_by_two_closed_form():
    """H_d = [[a, b], [b, c]]: U = [[sqrt(c/det), -b/sqrt(c det)], [0, 1/sqrt(c)]]."""
    a, b, c = 5.0, -2.0, 3.0
    det = a * c - b * b
    u = O.inverse_hessian_factor(np.array([[a, b], [b, c]]))
    want = np.array([[np.sqrt(c / det), -b / np.sqrt(c * det)], [0.0, 1.0 / np.sqrt(c)]])
    np.testing.assert_allclose(u, want, rtol=1e-14)


def test_u_of_diagonal_is_inverse_sqrt():
    h = np.diag([4.0, 9.0, 0.25, 16.0])
    np.testing.assert_allclose(O.inverse_hessian_factor(h), np.diag([0.5, 1 / 3, 2.0, 0.25]), rtol=1e-15)


def test_u_properties_and_two_step_identity():
    """U upper, U_jj > 0, U^T U H_d = I; and J inv(chol(J H_d J)) J is the same U
    (the positive-diagonal Cholesky factor is unique)."""
    d = 40
    a = RNG.standard_normal((200, d)) @ np.diag(1.0 / np.arange(1, d + 1))
    hd, _ = O.damp(2 * a.T @ a, 0.01)
    u = O.inverse_hessian_factor(hd)
    assert np.all(np.tril(u, -1) == 0) and np.all(np.diag(u) > 0)
    np.testing.assert_allclose(u.T @ u @ hd, np.eye(d), atol=1e-9)
    j = np.eye(d)[::-1]
    m = np.linalg.cholesky(j @ hd @ j)
    np.testing.assert_allclose(j @ np.linalg.inv(m) @ j, u, rtol=1e-9, atol=1e-12)


def test_u_not_positive_definite_raises():
    with pytest.raises(np.linalg.LinAlgError):
        O.inverse_hessian_factor(np.array([[1.0, 2.0], [2.0, 1.0]]))
    h0 = O.hessian(np.zeros((8, 4), np.float16))
    with pytest.raises(np.linalg.LinAlgError):
        O.inverse_hessian_factor(O.damp(h0, 0.01)[0])


# ---------------------------------------------------------------------------
# grid (stated reading; the hand cases are derived in tests/golden/grid_cases.txt)
# ---------------------------------------------------------------------------
def _frac(s):
    return float(Fraction(s))


def _grid_cases(golden_dir):
    with open(os.path.join(golden_dir, "grid_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, vals, s, z, codes, deq = [p.strip() for p in line.split("|")]
            grid, bits = head.split()
            yield (grid, int(bits), [_frac(v) for v in vals.split()], _frac(s), int(z),
                   [int(c) for c in codes.split()], [_frac(v) for v in deq.split()])


def test_grid_hand_cases(golden_dir):
    n = 0
    for grid, bits, vals, s, z, codes, deq in _grid_cases(golden_dir):
        v = np.array([vals])
        gs, gz, maxq = O.fit_grid(v, bits, grid)
        assert gs[0] == pytest.approx(s, rel=1e-14) and gz[0] == z
        r = O.rtn_quantize(v, bits, grid, 0)
        assert list(r.codes[0]) == codes
        np.testing.assert_allclose(r.w_hat[0], deq, rtol=1e-14, atol=1e-15)
        n += 1
    assert n == 8


def test_boundary_distance():
    p = np.array([0.2, 0.5004, 2.49, 15.7, -3.0])
    np.testing.assert_allclose(O.boundary_distance(p, 15), [0.3, 0.0004, 0.01, 1.2, 3.5], atol=1e-12)


# ---------------------------------------------------------------------------
# the column loop
# ---------------------------------------------------------------------------
def _correlated_layer(m, d, n, seed, outlier=True):
    rng = np.random.default_rng(seed)
    a = np.diag(1.0 / np.arange(1, d + 1)) @ np.linalg.qr(rng.standard_normal((d, d)))[0].T
    if outlier:
        a[:, rng.integers(d)] *= 8
    x = (rng.standard_normal((n, d)) @ a).astype(np.float16)
    w = (rng.standard_normal((m, d)) * 0.02).astype(np.float32)
    return w.astype(np.float64), x


@pytest.mark.parametrize("group,grid,bits", [(0, "asym", 4), (8, "asym", 3), (16, "ternary", 2), (0, "asym", 2),
                                             (8, "sym", 3), (0, "sym", 4)])
def test_rtn_reduction_when_h_is_scaled_identity(group, grid, bits):
    """XX^T = cI (Hadamard tokens): U is diagonal, nothing propagates, so GPTQ's
    codes equal round-to-nearest exactly, per row and per group."""
    n, d, m = 128, 32, 20
    x = _sylvester(n)[:, :d].astype(np.float16)
    w = RNG.standard_normal((m, d)) * 0.02
    res, h, u, _ = O.quantize_layer(w, x, bits, grid, group, block=8)
    np.testing.assert_array_equal(np.triu(u, 1), 0)
    rtn = O.rtn_quantize(w, bits, grid, group)
    np.testing.assert_array_equal(res.codes, rtn.codes)
    np.testing.assert_allclose(res.w_hat, rtn.w_hat, rtol=1e-15)


def test_single_column_is_rtn_with_closed_form_loss():
    """d = 1: GPTQ = RTN and ||(W - W_hat)X^T||^2 = sum_r (w_r - q_r)^2 sum_t x_t^2."""
    x = RNG.standard_normal((50, 1)).astype(np.float16)
    w = RNG.standard_normal((6, 1)) * 0.02
    res, h, _, _ = O.quantize_layer(w, x, 4, "asym", 0, block=1)
    rtn = O.rtn_quantize(w, 4, "asym", 0)
    np.testing.assert_array_equal(res.codes, rtn.codes)
    sx2 = float(np.sum(x.astype(np.float64) ** 2))
    want = float(np.sum((w - res.w_hat) ** 2)) * sx2
    assert O.layer_loss(w, res.w_hat, h) == pytest.approx(want, rel=1e-13)
    assert O.layer_loss_tokens(w, res.w_hat, x) == pytest.approx(want, rel=1e-13)


def test_two_column_closed_form():
    """d = 2, after column 1: w~2 = w2 + (H_d12/H_d22)(w1 - q1), and column 1's
    OBS increment is e1^2/2 = (w1 - q1)^2 det(H_d) / (2 H_d22)."""
    x = (RNG.standard_normal((40, 2)) @ np.array([[1.0, 0.6], [0.0, 0.8]])).astype(np.float16)
    w = RNG.standard_normal((5, 2)) * 0.05
    res, h, u, lam = O.quantize_layer(w, x, 3, "asym", 0, block=2)
    hd = h + lam * np.eye(2)
    s, z = res.scales[:, 0], res.zeros[:, 0]
    q1 = res.w_hat[:, 0]
    w2_updated = (res.p[:, 1] - z) * s
    np.testing.assert_allclose(w2_updated, w[:, 1] + hd[0, 1] / hd[1, 1] * (w[:, 0] - q1), rtol=1e-12)
    det = hd[0, 0] * hd[1, 1] - hd[0, 1] ** 2
    np.testing.assert_allclose(0.5 * res.err[:, 0] ** 2, (w[:, 0] - q1) ** 2 * det / (2 * hd[1, 1]), rtol=1e-12)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("block", [1, 2, 6])
def test_least_squares_resolve_at_every_step(seed, block):
    """Tiny layers (m <= 2, d <= 6, 2-bit): at every step j, with columns < j
    fixed to their quantized values q, the weight the oracle rounds equals the
    explicit least-squares re-solve of the remaining weights,
        w~_F = w_F + H_FF^-1 H_FP (w_P - q_P),   F = {j..}, P = {..j-1},
    the minimiser of (v - w) H_d (v - w)^T over v_F."""
    rng = np.random.default_rng(seed)
    m, d = 2, 6
    w, x = _correlated_layer(m, d, 60, seed)
    w = w * 8
    res, h, u, lam = O.quantize_layer(w, x, 2, "asym", 0, block=block)
    hd = h + lam * np.eye(d)
    for j in range(1, d):
        f, p = slice(j, d), slice(0, j)
        corr = np.linalg.solve(hd[f, f], hd[f, p] @ (w[:, p] - res.w_hat[:, p]).T).T
        w_tilde_j = (w[:, f] + corr)[:, 0]
        got = (res.p[:, j] - res.zeros[:, 0]) * res.scales[:, 0]
        np.testing.assert_allclose(got, w_tilde_j, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("seed", range(4))
def test_group_grid_is_fitted_on_updated_weights(seed):
    """At a group's first column j0 the grid is fitted to the current weights,
    which are the least-squares re-solve given the quantized columns < j0 (not
    the original weights): its range is that of w~_[j0, j0+g)."""
    d, g = 8, 4
    w, x = _correlated_layer(3, d, 80, 50 + seed)
    w = w * 6
    res, h, u, lam = O.quantize_layer(w, x, 3, "asym", g, block=g)
    hd = h + lam * np.eye(d)
    f, p = slice(g, d), slice(0, g)
    w_tilde = w[:, f] + np.linalg.solve(hd[f, f], hd[f, p] @ (w[:, p] - res.w_hat[:, p]).T).T
    lo = np.minimum(w_tilde.min(axis=1), 0.0)
    hi = np.maximum(w_tilde.max(axis=1), 0.0)
    np.testing.assert_allclose(res.scales[:, 1], (hi - lo) / 7, rtol=1e-11)
    assert not np.allclose(res.scales[:, 1], (np.maximum(w[:, f].max(1), 0) - np.minimum(w[:, f].min(1), 0)) / 7,
                           rtol=1e-6)


def test_obs_loss_identity():
    """sum_{r,j} e_rj^2 / 2 = ||(W - W_hat)X^T||^2 + (lambda/2) ||W - W_hat||^2
    (the OBS increments of the damped objective telescope)."""
    w, x = _correlated_layer(12, 48, 400, 7)
    res, h, u, lam = O.quantize_layer(w, x, 3, "asym", 16, block=16)
    lhs = float(np.sum(res.obs_loss))
    rhs = O.layer_loss_tokens(w, res.w_hat, x) + 0.5 * lam * float(np.sum((w - res.w_hat) ** 2))
    assert lhs == pytest.approx(rhs, rel=1e-10)
    assert O.layer_loss(w, res.w_hat, h) == pytest.approx(O.layer_loss_tokens(w, res.w_hat, x), rel=1e-11)


@pytest.mark.parametrize("group", [0, 32])
def test_block_size_invariance(group):
    """Lazy batching changes no result: B in {1, 7, 32, 128, d} and the
    unblocked form give the same codes and W_hat."""
    w, x = _correlated_layer(16, 128, 600, 11)
    h = O.hessian(x)
    u = O.inverse_hessian_factor(O.damp(h)[0])
    ref = O.gptq_quantize(w, u, 4, "asym", group, blocked=False)
    blocks = [1, 32, 128] + ([7, 128] if group == 0 else [64])
    for b in blocks:
        r = O.gptq_quantize(w, u, 4, "asym", group, block=b)
        np.testing.assert_array_equal(r.codes, ref.codes)
        np.testing.assert_allclose(r.w_hat, ref.w_hat, rtol=1e-12, atol=1e-15)


def test_scale_invariance_of_codes():
    """X -> 2^k X (exact in fp16) multiplies H by 4^k and leaves every code unchanged."""
    w, x = _correlated_layer(10, 64, 300, 3)
    r1, h1, _, _ = O.quantize_layer(w, x, 3, "asym", 0, block=32)
    r2, h2, _, _ = O.quantize_layer(w, (x.astype(np.float32) * 4).astype(np.float16), 3, "asym", 0, block=32)
    np.testing.assert_array_equal(h2, 16 * h1)
    np.testing.assert_array_equal(r1.codes, r2.codes)


@pytest.mark.parametrize("bits,group", [(3, 0), (4, 0), (3, 32), (2, 32)])
def test_gptq_beats_rtn_on_correlated_inputs(bits, group):
    w, x = _correlated_layer(32, 128, 800, 5)
    res, h, _, _ = O.quantize_layer(w, x, bits, "asym", group)
    rtn = O.rtn_quantize(w, bits, "asym", group)
    assert O.layer_loss(w, res.w_hat, h) < O.layer_loss(w, rtn.w_hat, h)


def test_brute_force_bound_and_rtn_comparison():
    """1 x 4 and 1 x 5 layers, 2-bit: enumerate every code vector on the same
    grid; the optimum is never above GPTQ (a sanity bound, not a pin of codes)."""
    wins = 0
    for seed in range(10):
        d = 4 + seed % 2
        w, x = _correlated_layer(1, d, 40, 100 + seed)
        w = w * 10
        res, h, _, _ = O.quantize_layer(w, x, 2, "asym", 0, block=d)
        s, z = res.scales[0, 0], res.zeros[0, 0]
        best = min(O.layer_loss(w, s * (np.array([c]) - z), h) for c in itertools.product(range(4), repeat=d))
        lg = O.layer_loss(w, res.w_hat, h)
        assert best <= lg * (1 + 1e-12)
        wins += lg <= O.layer_loss(w, O.rtn_quantize(w, 2, "asym", 0).w_hat, h) * (1 + 1e-12)
    assert wins >= 7


# ---------------------------------------------------------------------------
# follow mode (plants mistakes in the oracle's input, on the CPU)
# ---------------------------------------------------------------------------
def test_follow_mode_counts():
    """Mistakes are planted in the last column, so no later column of the row
    depends on them: one off-by-two code (hard) and one code moved across a
    boundary that p lies within 1e-3 of (band)."""
    m, d = 3000, 32
    w, x = _correlated_layer(m, d, 400, 9)
    res, h, u, _ = O.quantize_layer(w, x, 3, "asym", 32, block=32)
    same = O.gptq_quantize(w, u, 3, "asym", 32, block=32, follow_codes=res.codes, follow_zeros=res.zeros)
    assert same.band_mismatch == 0 and same.hard_mismatch == 0
    np.testing.assert_array_equal(same.codes, res.codes)
    planted = res.codes.copy()
    last = d - 1
    r = int(np.argmax(res.dist[:, last]))
    planted[r, last] = (planted[r, last] + 2) % 8
    dist = res.dist[:, last].copy()
    dist[r] = 9.0
    r2 = int(np.argmin(dist))
    assert dist[r2] < 1e-3
    p = res.p[r2, last]
    lowc = int(np.floor(p))
    planted[r2, last] = lowc if res.codes[r2, last] == lowc + 1 else lowc + 1
    f = O.gptq_quantize(w, u, 3, "asym", 32, block=32, follow_codes=planted, follow_zeros=res.zeros)
    assert f.hard_mismatch == 1 and f.band_mismatch == 1
    assert f.hard_positions == [(r, last)]
    np.testing.assert_array_equal(f.codes, planted)


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------
def _pack_cases(golden_dir):
    with open(os.path.join(golden_dir, "pack_vectors.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            bits, n, rule = int(parts[0]), int(parts[1]), parts[2]
            mod = int(rule.replace("jmod", ""))
            yield bits, np.arange(n) % mod, [int(v, 16) for v in parts[3:]]


def test_pack_hand_vectors(golden_dir):
    cases = list(_pack_cases(golden_dir))
    assert len(cases) == 4
    for bits, codes, words in cases:
        got = O.pack_codes(codes[None, :], bits)
        assert [int(v) for v in got[0]] == words


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_round_trip(bits):
    d = 64 if bits != 3 else 96
    codes = RNG.integers(0, 1 << bits, size=(7, d))
    np.testing.assert_array_equal(O.unpack_codes(O.pack_codes(codes, bits), bits, d), codes)


@pytest.mark.parametrize("group", [0, 8])
def test_zero_point_follow_at_the_all_zero_tie(group):
    """An all-zero row (or group) takes the grid (-1, +1): -lo/s = maxq/2
    exactly, a half-integer, which finite precision rounds either way. Follow
    mode takes the other neighbour as a band mismatch (judged with the lo the
    fit uses, -1, not the raw 0), and a zero point two steps away as hard."""
    m, d, bits = 3, 16, 4
    w = RNG.standard_normal((m, d)) * 0.1
    w[1] = 0.0
    u = np.eye(d)
    base = O.gptq_quantize(w, u, bits, "asym", group, block=8)
    assert base.zeros[1, 0] in (7, 8)
    other = base.zeros.copy()
    other[1, :] = 15 - base.zeros[1, :]
    res = O.gptq_quantize(w, u, bits, "asym", group, block=8, follow_codes=base.codes, follow_zeros=other)
    ng = other.shape[1]
    assert (res.zero_band_mismatch, res.zero_hard_mismatch) == (ng, 0)
    assert np.all(res.zeros[1] == other[1])
    far = base.zeros.copy()
    far[0, 0] += 2
    res2 = O.gptq_quantize(w, u, bits, "asym", group, block=8, follow_zeros=far)
    assert res2.zero_hard_mismatch == 1


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_symmetric_grid_properties(bits):
    """Symmetric grid: the zero point is the integer 2^(b-1), so code z is
    exactly 0 and 0 rounds to it; every value inside the levels' range rounds
    to within s/2; the extreme level -z s lies within one step of -max|v|."""
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((5, 40)) * 0.3
    s, z, maxq = O.fit_grid(v, bits, "sym")
    assert np.all(z == 1 << (bits - 1))
    a = np.max(np.abs(v), axis=1)
    np.testing.assert_allclose(s, 2 * a / maxq, rtol=1e-15)
    r = O.rtn_quantize(np.concatenate([v, np.zeros((5, 8))], axis=1), bits, "sym", 0)
    assert np.all(r.codes[:, 40:] == z[:, None]) and np.all(r.w_hat[:, 40:] == 0.0)
    inside = (v >= -z[:, None] * s[:, None]) & (v <= (maxq - z)[:, None] * s[:, None])
    err = np.abs(r.w_hat[:, :40] - v)
    assert np.all(err[inside] <= (s[:, None] / 2 * np.ones_like(v))[inside] * (1 + 1e-12))
    assert np.all(-z * s <= -a) and np.all(-z * s >= -a - s)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_asymmetric_grid_properties(bits):
    """Asymmetric min-max grid, checked by what a uniform grid over the widened
    range [min(v, 0), max(v, 0)] must satisfy rather than by its formula: the
    zero point is an integer code in [0, maxq] and that code is exactly 0; the
    lowest and highest levels lie within half a step of the range's ends; every
    value in the range rounds to within half a step; the step is the smallest
    that covers the range with maxq + 1 levels (s maxq = range); and when both
    ends are levels of such a grid (lo = -k t, hi = (maxq - k) t) they are
    reproduced exactly."""
    rng = np.random.default_rng(100 + bits)
    v = rng.standard_normal((6, 48)) * 0.05
    v[1] = np.abs(v[1])          # all >= 0: lo = 0
    v[2] = -np.abs(v[2])         # all <= 0: hi = 0
    v[3, :4] = [3.0, -0.1, 0.2, -0.4]   # a strong outlier
    s, z, maxq = O.fit_grid(v, bits, "asym")
    assert np.all((z >= 0) & (z <= maxq)) and z.dtype.kind == "i"
    lo = np.minimum(v.min(axis=1), 0.0)
    hi = np.maximum(v.max(axis=1), 0.0)
    np.testing.assert_allclose(s * maxq, hi - lo, rtol=1e-14)
    assert np.all(np.abs(-z * s - lo) <= s / 2 * (1 + 1e-12))
    assert np.all(np.abs((maxq - z) * s - hi) <= s / 2 * (1 + 1e-12))
    assert z[1] == 0 and z[2] == maxq
    r = O.rtn_quantize(np.concatenate([v, np.zeros((6, 8))], axis=1), bits, "asym", 0)
    assert np.all(r.codes[:, 48:] == z[:, None]) and np.all(r.w_hat[:, 48:] == 0.0)
    err = np.abs(r.w_hat[:, :48] - v)
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))
    # ends on the grid: lo = -k t, hi = (maxq - k) t with t a power of two
    for k in (0, 1, maxq // 2, maxq - 1):
        t = 2.0 ** -6
        vv = np.array([[-k * t, (maxq - k) * t, 0.3 * t]])
        s1, z1, _ = O.fit_grid(vv, bits, "asym")
        q = O.rtn_quantize(vv, bits, "asym", 0)
        assert s1[0] == t and z1[0] == k
        assert q.w_hat[0, 0] == -k * t and q.w_hat[0, 1] == (maxq - k) * t


def test_hessian_factor_definition_and_relations():
    """R upper with a positive diagonal and R R^T = H_d; R^-1 equals the
    inverse-Hessian factor U (both are the unique positive-diagonal triangular
    factors); a diagonal H_d gives R = diag(sqrt(h)); the 2 x 2 closed form
    R = [[sqrt(a - b^2/c), b/sqrt(c)], [0, sqrt(c)]] for H_d = [[a, b], [b, c]]."""
    rng = np.random.default_rng(31)
    for d in (1, 2, 7, 40):
        x = rng.standard_normal((3 * d + 5, d)) @ rng.standard_normal((d, d))
        hd, _ = O.damp(O.hessian(x), 0.01)
        r = O.hessian_factor(hd)
        assert np.allclose(np.tril(r, -1), 0.0) and np.all(np.diag(r) > 0)
        np.testing.assert_allclose(r @ r.T, hd, rtol=1e-12, atol=1e-12 * np.abs(hd).max())
        u = O.inverse_hessian_factor(hd)
        np.testing.assert_allclose(np.linalg.inv(r), u, rtol=1e-9, atol=1e-12 * np.abs(u).max())
    h = np.diag([4.0, 9.0, 0.25])
    np.testing.assert_array_equal(O.hessian_factor(h), np.diag([2.0, 3.0, 0.5]))
    a, b, c = 5.0, 2.0, 4.0
    r2 = O.hessian_factor(np.array([[a, b], [b, c]]))
    np.testing.assert_allclose(r2, [[np.sqrt(a - b * b / c), b / np.sqrt(c)], [0.0, np.sqrt(c)]], rtol=1e-15)
    with pytest.raises(np.linalg.LinAlgError):
        O.hessian_factor(np.array([[1.0, 2.0], [2.0, 1.0]]))


@pytest.mark.parametrize("d,block", [(300, 64), (257, 100), (64, 64), (5, 2)])
def test_hessian_factor_blocked_path(d, block):
    """The blocked path (taken at widths whose d * d reaches 2^31) on small
    matrices, ragged last blocks included: R upper with a positive diagonal
    and R R^T = H_d (which fix R uniquely), the diagonal and 2 x 2 closed forms,
    the unblocked path's R within rounding, and LinAlgError on an indefinite
    matrix."""
    rng = np.random.default_rng(d + block)
    x = rng.standard_normal((3 * d + 5, d)) @ rng.standard_normal((d, d))
    hd, _ = O.damp(O.hessian(x), 0.01)
    r = O.hessian_factor(hd, block=block)
    assert np.all(np.tril(r, -1) == 0.0) and np.all(np.diag(r) > 0)
    np.testing.assert_allclose(r @ r.T, hd, rtol=1e-12, atol=1e-12 * np.abs(hd).max())
    np.testing.assert_allclose(r, O.hessian_factor(hd), rtol=1e-9, atol=1e-12 * np.abs(r).max())
    np.testing.assert_array_equal(O.hessian_factor(np.diag([4.0, 9.0, 0.25]), block=2), np.diag([2.0, 3.0, 0.5]))
    a, b, c = 5.0, 2.0, 4.0
    np.testing.assert_allclose(O.hessian_factor(np.array([[a, b], [b, c]]), block=1),
                               [[np.sqrt(a - b * b / c), b / np.sqrt(c)], [0.0, np.sqrt(c)]], rtol=1e-15)
    with pytest.raises(np.linalg.LinAlgError):
        O.hessian_factor(np.array([[1.0, 2.0, 0.0], [2.0, 1.0, 0.0], [0.0, 0.0, 1.0]]), block=1)


def test_large_width_forms(monkeypatch):
    """From BLAS_SYRK_MAX entries on (the fc2 width with the real limit),
    hessian takes a general product of an explicit copy of X^T and
    hessian_factor the blocked algorithm; with the limit lowered, both on a
    small input against the plain forms."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 90)).astype(np.float16)
    h_plain = O.hessian(x)
    r_plain = O.hessian_factor(O.damp(h_plain, 0.01)[0])
    import oracle.gptq_oracle as OM  # the module whose global the two functions read
    monkeypatch.setattr(OM, "BLAS_SYRK_MAX", 90 * 90)
    calls = []
    blocked = OM._cholesky_lower_blocked
    monkeypatch.setattr(OM, "_cholesky_lower_blocked", lambda a, b, p=None: calls.append(b) or blocked(a, b, p))
    h = O.hessian(x)
    np.testing.assert_allclose(h, h_plain, rtol=1e-13, atol=1e-12)
    assert np.all(h == h.T)
    hd = O.damp(h, 0.01)[0]
    r = O.hessian_factor(hd)
    assert np.all(np.tril(r, -1) == 0.0) and np.all(np.diag(r) > 0)
    np.testing.assert_allclose(r @ r.T, hd, rtol=1e-12, atol=1e-12 * np.abs(hd).max())
    np.testing.assert_allclose(r, r_plain, rtol=1e-9, atol=1e-12 * np.abs(r).max())
    assert calls == [4096]  # the factor took the blocked path


@pytest.mark.parametrize("group", [16, 48, 96, 192])
def test_groups_not_aligned_to_the_block_are_block_size_invariant(group):
    """Group sizes that neither divide the 128-column block nor are multiples of
    it: a group fitted at its first column sees every earlier update whatever
    the block size, so the blocked loop at B in {1, 7, 32, 128} and the
    unblocked loop give the same codes, grids and W_hat. (A fit on the
    partially updated weights past the block end would depend on B.)"""
    rng = np.random.default_rng(group)
    m, d = 6, 384
    x = rng.standard_normal((4 * d, d)) @ (rng.standard_normal((d, d)) / np.sqrt(d) + np.eye(d))
    hd, _ = O.damp(O.hessian(x), 0.01)
    u = O.inverse_hessian_factor(hd)
    w = rng.standard_normal((m, d)) * 0.05
    ref = O.gptq_quantize(w, u, 3, "asym", group, blocked=False)
    for block in (1, 7, 32, 128):
        r = O.gptq_quantize(w, u, 3, "asym", group, block=block)
        near = ref.dist < 1e-9
        assert np.all((r.codes == ref.codes) | near), block
        np.testing.assert_allclose(r.scales, ref.scales, rtol=1e-10)
        np.testing.assert_array_equal(r.zeros, ref.zeros)
        np.testing.assert_allclose(r.w_hat, ref.w_hat, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("group", [16, 96])
def test_unaligned_groups_reduce_to_rtn_when_h_is_diagonal(group):
    """With a diagonal H no error propagates: the codes are round-to-nearest
    on groups of the original weights, for unaligned group sizes too."""
    rng = np.random.default_rng(5)
    m, d = 5, 384
    hd = np.diag(rng.uniform(0.5, 2.0, d))
    u = O.inverse_hessian_factor(hd)
    w = rng.standard_normal((m, d)) * 0.05
    g = O.gptq_quantize(w, u, 4, "asym", group)
    r = O.rtn_quantize(w, 4, "asym", group)
    np.testing.assert_array_equal(g.codes, r.codes)
    np.testing.assert_array_equal(g.scales, r.scales)
