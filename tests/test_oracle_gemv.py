"""Pins of the oracle's dequantizing matrix-vector product (y = W_hat x read
from the packed codes): hand vectors from the packing fixtures, an exact
rational evaluation of the per-group regrouping, and agreement with the
quantizer's own W_hat."""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.abspath(__file__))


def _golden_rows():
    rows = []
    for line in open(os.path.join(ROOT, "golden", "pack_vectors.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        bits, n, rule = int(line[0]), int(line[1]), line[2]
        words = np.array([int(w, 16) for w in line[3:]], dtype=np.uint32)
        mod = int(rule.replace("jmod", ""))
        rows.append((bits, n, mod, words))
    return rows


@pytest.mark.parametrize("row", range(4))
def test_hand_vectors(row):
    """Codes j mod K packed by hand: with s = 1 and z = 0, y against e_k is code
    k, and y against the ones vector is the sum of the codes."""
    bits, n, mod, words = _golden_rows()[row]
    w = words[None, :]
    s = np.ones((1, 1))
    z = np.zeros((1, 1), dtype=np.int64)
    for k in (0, n // 2, n - 1):
        e = np.zeros(n)
        e[k] = 1.0
        assert O.dequant_matvec(w, s, z, bits, 0, e)[0] == k % mod
    assert O.dequant_matvec(w, s, z, bits, 0, np.ones(n))[0] == sum(j % mod for j in range(n))


def test_grouped_sum_in_exact_rationals():
    """y_r = sum_g s_rg (sum_{j in g} c_rj x_j - z_rg sum_{j in g} x_j), evaluated
    in exact rationals with pure-Python loops on a 3-bit, g32 layer."""
    rng = np.random.default_rng(5)
    m, d, g, bits = 3, 96, 32, 3
    c = rng.integers(0, 8, (m, d))
    s = rng.uniform(0.001, 0.01, (m, d // g))
    z = rng.integers(0, 8, (m, d // g))
    x = rng.standard_normal(d)
    y = O.dequant_matvec(O.pack_codes(c, bits), s, z, bits, g, x)
    for r in range(m):
        exact = Fraction(0)
        for k in range(d // g):
            cx = sum(Fraction(int(c[r, j])) * Fraction(x[j]) for j in range(k * g, (k + 1) * g))
            sx = sum(Fraction(x[j]) for j in range(k * g, (k + 1) * g))
            exact += Fraction(s[r, k]) * (cx - int(z[r, k]) * sx)
        assert y[r] == pytest.approx(float(exact), rel=1e-13, abs=1e-15)


@pytest.mark.parametrize("group,grid,bits", [(0, "asym", 4), (16, "asym", 3), (16, "ternary", 2)])
def test_matches_the_quantizers_w_hat(group, grid, bits):
    rng = np.random.default_rng(group + bits)
    m, d, n = 6, 64, 200
    x_cal = rng.standard_normal((n, d)).astype(np.float16)
    w = rng.standard_normal((m, d)) * 0.05
    res, _, _, _ = O.quantize_layer(w, x_cal, bits, grid, group, block=16)
    v = rng.standard_normal(d)
    y = O.dequant_matvec(O.pack_codes(res.codes, bits), res.scales, res.zeros, bits, group, v)
    np.testing.assert_allclose(y, res.w_hat @ v, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("bits,group", [(3, 16), (4, 32)])
def test_group_index_matches_the_act_order_quantizers_w_hat(bits, group):
    """Act-order without static groups: the codes stay in natural column order
    and g_idx names every column's group; y from (codes, scales, zeros, g_idx)
    equals the ordered quantizer's own W_hat times x."""
    rng = np.random.default_rng(bits * group)
    m, d, n = 5, 64, 300
    x_cal = (rng.standard_normal((n, d)) * np.linspace(0.2, 3.0, d)).astype(np.float16)
    w = rng.standard_normal((m, d)) * 0.05
    res, g_idx, perm, _, _, _ = O.quantize_layer_act_order(w, x_cal, bits, "asym", group, static_groups=False,
                                                           block=16)
    assert not np.array_equal(g_idx, np.arange(d) // group)   # the groups are not natural runs
    v = rng.standard_normal(d)
    y = O.dequant_matvec(O.pack_codes(res.codes, bits), res.scales, res.zeros, bits, group, v, g_idx=g_idx)
    np.testing.assert_allclose(y, res.w_hat @ v, rtol=1e-12, atol=1e-15)
    # columns sorted by group (stable) are runs of `group` columns: the natural
    # grouped product of the sorted codes against x in that order is the same y
    order = np.argsort(g_idx, kind="stable")
    assert np.array_equal(g_idx[order], np.arange(d) // group)
    y_sorted = O.dequant_matvec(O.pack_codes(res.codes[:, order], bits), res.scales, res.zeros, bits, group, v[order])
    np.testing.assert_allclose(y_sorted, y, rtol=1e-12, atol=1e-15)
