"""Plain fp64 CPU oracle of the GPTQ layer-wise quantization hot path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The GPU library never calls it, and the oracle never imports the GPU
package: the two share no code, no tables and no helpers. Inputs reach both
sides only through the seeded generators, which hold none of the method's
arithmetic.

Sources (cited by page title and section):

* [FDE] "GPTQ: Accurate Post-Training Quantization for Generative Pre-trained
  Transformers", breakdown by FDE Interviews -- section 01 "The paper in one
  minute" and the figure "Quantize a column, correct the rest (Section 4)",
  steps 1-4.
* [NUB] "[Paper Review] GPTQ: Accurate Post-Training Quantization for
  Generative Pre-trained Transformers" (nubint) -- "Proposed method" and
  "Key findings".
* [ZLY] "GPTQ：用于生成式预训练 Transformer 的准确训练后量化" (zhiliyouxian
  blog) -- "数学基础 / 问题公式化" (the objective), "超参数选择" and "实践指南"
  (defaults, the desc_act option).
* [CSDN] "GPTQ量化参数搜索工具：自动寻找最优配置" -- its parameter table, which
  names --desc_act and --static_groups.

Everything is numpy float64. fp16/fp32 inputs are upcast exactly. Library
primitives (matmul, numpy.linalg.cholesky, numpy.linalg.inv) serve as single
steps; there is no blocking, fusion or reordering beyond what the method states
(the lazy 128-column blocks are part of the method, and an unblocked variant is
kept beside the blocked one).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* H is unnormalised, H = 2 X^T X with X token-major [N, d] (the same d x d
  matrix as 2 X X^T with X = [d, N]).
* Damping is relative: lambda = damp * mean(diag H), added to the diagonal.
* The grid is asymmetric min-max (range widened to include 0), with an integer
  zero point z = rint(-lo/s); or ternary {-s, 0, +s} with s = max|v|; or
  symmetric min-max, s = 2 max|v| / maxq with z = (maxq + 1) / 2.
* Act-order quantizes the columns in descending H_jj (ties in index order);
  static groups keep each column on the grid of its natural group, fitted on
  the original weights before the loop (see the act-order section).
* Where rounding decides an integer at an exact tie (a zero point at a
  half-integer), follow mode takes the other implementation's neighbour.
* A per-row grid is fitted once on the original row; a per-group grid is
  fitted at the group's first column on the current, updated weights.
* Rounding is IEEE round-half-to-even (numpy.rint).
* Codes are packed LSB-first into uint32 words, row by row.

Parity status of each function is stated in its docstring. The grid
conventions (fit_grid, its asymmetric, ternary and symmetric forms), the
act-order key (act_order_perm) and the static-group rule (static_group_grids)
are "parity unpinned" against the pages: the pages never define them, so only
the stated readings and the invariants the tests check pin them.
"""

from __future__ import annotations

import numpy as np

GRID_ASYM = "asym"
GRID_TERNARY = "ternary"
GRID_SYM = "sym"


# ---------------------------------------------------------------------------
# Step 1: the Hessian of the layer-wise objective.
# ---------------------------------------------------------------------------
# numpy hands products of the form x.T @ x, and LAPACK its Cholesky updates,
# to the BLAS symmetric rank-k update, which in the OpenBLAS build here crashes
# once the output has 2^31 entries (d >= 46341: the OPT-175B fc2 width). From
# that size on, hessian and hessian_factor take the same results another way.
BLAS_SYRK_MAX = 2 ** 31


def hessian(x_chunks) -> np.ndarray:
    """H = 2 * sum_c X_c^T X_c in fp64 over token-major chunks X_c [n_c, d].

    [FDE] "The paper in one minute": the least-squares objective for one layer
    has curvature H = 2XX^T computed from the calibration inputs; also the
    caption of the figure "Quantize a column, correct the rest".
    fp16 x fp16 products are exact in fp64; only the summation rounds.
    """
    if isinstance(x_chunks, np.ndarray):
        x_chunks = [x_chunks]
    h = None
    for xc in x_chunks:
        x = np.asarray(xc, dtype=np.float64)
        # from BLAS_SYRK_MAX on, a general product of an explicit copy of x^T
        part = x.T @ x if x.shape[1] ** 2 < BLAS_SYRK_MAX else np.ascontiguousarray(x.T) @ x
        h = part if h is None else h + part
    return 2.0 * h


def layer_loss_tokens(w, w_hat, x_chunks) -> float:
    """||(W - W_hat) X^T||_F^2 evaluated directly over the tokens.

    [ZLY] "问题公式化": minimise ||Wx - W_hat x||^2 over the calibration inputs;
    [FDE] "The paper in one minute": keep the layer's outputs on the
    calibration set unchanged.
    """
    if isinstance(x_chunks, np.ndarray):
        x_chunks = [x_chunks]
    delta = np.asarray(w, np.float64) - np.asarray(w_hat, np.float64)
    total = 0.0
    for xc in x_chunks:
        out = delta @ np.asarray(xc, np.float64).T
        total += float(np.sum(out * out))
    return total


def layer_loss(w, w_hat, h) -> float:
    """||(W - W_hat) X^T||_F^2 through the undamped H = 2 X^T X.

    Since Delta X^T X Delta^T = 1/2 Delta H Delta^T, this equals
    layer_loss_tokens exactly in exact arithmetic (the tests check both).
    """
    delta = np.asarray(w, np.float64) - np.asarray(w_hat, np.float64)
    return 0.5 * float(np.sum((delta @ np.asarray(h, np.float64)) * delta))


# ---------------------------------------------------------------------------
# Step 2: dampening.
# ---------------------------------------------------------------------------
def damp(h, percdamp: float = 0.01) -> tuple[np.ndarray, float]:
    """Return (H + lambda*I, lambda) with lambda = percdamp * mean(diag H).

    [NUB] "Proposed method": a Cholesky reformulation and dampening keep the
    method numerically stable; [ZLY] "超参数选择": damp_percent = 0.01.
    Reading: the percentage is taken of the mean diagonal, the one scale H
    carries, so that the codes do not depend on the scale of H.
    """
    h = np.array(h, dtype=np.float64, copy=True)
    lam = percdamp * float(np.mean(np.diag(h)))
    h[np.diag_indices_from(h)] += lam
    return h, lam


# ---------------------------------------------------------------------------
# Step 3: upper Cholesky factor of the inverse Hessian.
# ---------------------------------------------------------------------------
def inverse_hessian_factor(h_damped) -> np.ndarray:
    """U upper triangular with positive diagonal and U^T U = H_d^{-1}.

    [FDE] figure "Quantize a column, correct the rest", step 2:
    U = chol(H^-1); section 01: the needed rows of the inverse Hessian come
    from a Cholesky decomposition. The definition is written out: invert H_d,
    take the (lower) Cholesky factor L of H_d^{-1} = L L^T, return U = L^T.
    Raises numpy.linalg.LinAlgError when H_d is not positive definite.
    """
    hd = np.asarray(h_damped, dtype=np.float64)
    np.linalg.cholesky(hd)  # raises when H_d itself is not positive definite
    hinv = np.linalg.inv(hd)
    hinv = 0.5 * (hinv + hinv.T)
    lower = np.linalg.cholesky(hinv)
    return np.triu(lower.T)


def hessian_factor(h_damped, block=None, progress=None) -> np.ndarray:
    """R upper triangular with positive diagonal and R R^T = H_d, so that
    R^-1 is the factor U of inverse_hessian_factor (U^T U = H_d^-1 gives
    H_d = U^-1 U^-T).

    [FDE] section 01: the needed rows of the inverse Hessian are taken from a
    Cholesky decomposition of the Hessian. The definition is written out with
    the reversal permutation J: L = chol(J H_d J) (lower), R = J L J.
    Raises numpy.linalg.LinAlgError when H_d is not positive definite. block:
    take L by the blocked algorithm with that block width (always used once
    d * d reaches BLAS_SYRK_MAX); progress(k, d), when given, is called after
    each of its column blocks (k columns done).
    """
    hd = np.asarray(h_damped, dtype=np.float64)
    d = hd.shape[0]
    a = np.ascontiguousarray(hd[::-1, ::-1])  # J H_d J
    if block is None and d * d < BLAS_SYRK_MAX:
        lower = np.linalg.cholesky(a)
    else:
        # from BLAS_SYRK_MAX on, the same factor by the blocked algorithm below
        lower = _cholesky_lower_blocked(a, block or 4096, progress)
    return np.triu(lower[::-1, ::-1])  # J L J


def _cholesky_lower_blocked(a, b, progress=None):
    """The lower Cholesky factor of the symmetric positive definite a, b
    columns at a time (the textbook right-looking block algorithm; a is
    overwritten): the diagonal block A11 = L11 L11^T (LAPACK), the block column
    below it L21 = A21 L11^-T (a solve with L11), and the rest of the lower
    triangle A22 -= L21 L21^T (general matrix products of explicit copies, one
    column block at a time)."""
    d = a.shape[0]
    for k0 in range(0, d, b):
        k1 = min(k0 + b, d)
        l11 = np.linalg.cholesky(a[k0:k1, k0:k1])
        a[k0:k1, k0:k1] = l11
        if k1 == d:
            if progress is not None:
                progress(k1, d)
            break
        l21 = np.linalg.solve(l11, a[k1:, k0:k1].T).T  # L11 L21^T = A21^T
        a[k1:, k0:k1] = l21
        l21c = np.ascontiguousarray(l21)
        for j0 in range(k1, d, b):
            j1 = min(j0 + b, d)
            # rows from j0 on: the lower triangle of the column block
            a[j0:, j0:j1] -= l21c[j0 - k1:] @ np.ascontiguousarray(l21c[j0 - k1:j1 - k1].T)
        if progress is not None:
            progress(k1, d)
    for k0 in range(0, d, b):  # the strict upper triangle (never written) to zero
        a[k0:k0 + b, k0 + 1:] = np.tril(a[k0:k0 + b, k0 + 1:], -1)
    return a


# ---------------------------------------------------------------------------
# Grid (quantizer). The pages only say "3/4-bit grid" and "ternary": the fit
# below is the stated reading (parity unpinned against the pages).
# ---------------------------------------------------------------------------
def maxq_of(bits: int, grid: str) -> int:
    if grid == GRID_TERNARY:
        return 2
    return (1 << bits) - 1


def fit_grid(v, bits: int, grid: str):
    """Scale and integer zero of a grid fitted to the rows of v.

    v: [m, k] values; returns (s [m] float64, z [m] int64, maxq).

    asym: lo = min(min v, 0), hi = max(max v, 0); lo = hi = 0 -> (-1, +1);
          s = (hi - lo) / maxq; z = rint(-lo / s).
    ternary: a = max|v| (0 -> 1); s = a; z = 1; maxq = 2 (levels -s, 0, +s).
    sym: a = max|v| (0 -> 1); s = 2a / maxq; z = (maxq + 1) / 2, the integer
         just above the midpoint of the codes, so that code z is exactly 0.
    [NUB] "Key findings": quantization down to 2-bit or ternary levels, with
    grouping, and compatibility with various grids; [FDE] figure step 1: round
    to the 3/4-bit grid.
    """
    v = np.asarray(v, dtype=np.float64)
    maxq = maxq_of(bits, grid)
    if grid == GRID_TERNARY:
        a = np.max(np.abs(v), axis=1)
        a = np.where(a == 0.0, 1.0, a)
        return a, np.ones(v.shape[0], dtype=np.int64), maxq
    if grid == GRID_SYM:
        a = np.max(np.abs(v), axis=1)
        a = np.where(a == 0.0, 1.0, a)
        return 2.0 * a / maxq, np.full(v.shape[0], (maxq + 1) // 2, dtype=np.int64), maxq
    if grid != GRID_ASYM:
        raise ValueError(f"unknown grid {grid!r}")
    lo = np.minimum(np.min(v, axis=1), 0.0)
    hi = np.maximum(np.max(v, axis=1), 0.0)
    both_zero = (lo == 0.0) & (hi == 0.0)
    lo = np.where(both_zero, -1.0, lo)
    hi = np.where(both_zero, 1.0, hi)
    s = (hi - lo) / maxq
    z = np.rint(-lo / s).astype(np.int64)
    return s, z, maxq


def boundary_distance(p, maxq: int) -> np.ndarray:
    """Distance (grid units) from p to the nearest decision boundary k + 1/2,
    0 <= k < maxq. Boundaries outside the clamp range do not exist."""
    b = np.clip(np.floor(p) + 0.5, 0.5, maxq - 0.5)
    return np.abs(p - b)


def follow_zero_points(v, s, z, fz, band: float):
    """Follow mode for the integer zero points of asymmetric grids fitted to the
    rows of v (scales s, the oracle's zero points z) against another
    implementation's zero points fz. A differing zero point is a band mismatch
    when it is the adjacent integer and -lo/s lies within `band` of the
    half-integer between the two (lo as the fit takes it: min(v, 0), or -1 when
    both ends are 0); anything else is a hard mismatch. Returns (the zero points
    to continue with, band count, hard count)."""
    v = np.asarray(v, dtype=np.float64)
    fz = np.asarray(fz).astype(np.int64).reshape(-1)
    lo = np.minimum(np.min(v, axis=1), 0.0)
    hi = np.maximum(np.max(v, axis=1), 0.0)
    lo = np.where((lo == 0.0) & (hi == 0.0), -1.0, lo)
    zr = -lo / s
    diff = fz != z
    near = np.abs(zr - (np.minimum(fz, z) + 0.5)) < band
    adj = np.abs(fz - z) == 1
    return (np.where(diff, fz, z), int(np.sum(diff & near & adj)), int(np.sum(diff & ~(near & adj))))


# ---------------------------------------------------------------------------
# Step 4: the column loop.
# ---------------------------------------------------------------------------
class QuantResult:
    """Outputs of one quantized layer (all numpy)."""

    def __init__(self, m, d, ngroups):
        self.codes = np.zeros((m, d), dtype=np.int64)
        self.w_hat = np.zeros((m, d), dtype=np.float64)
        self.err = np.zeros((m, d), dtype=np.float64)      # e_rj
        self.p = np.zeros((m, d), dtype=np.float64)        # pre-round value
        self.dist = np.zeros((m, d), dtype=np.float64)     # to nearest boundary
        self.scales = np.zeros((m, ngroups), dtype=np.float64)
        self.zeros = np.zeros((m, ngroups), dtype=np.int64)
        # follow-mode bookkeeping
        self.band_mismatch = 0
        self.hard_mismatch = 0
        self.hard_positions = []
        self.zero_band_mismatch = 0
        self.zero_hard_mismatch = 0

    @property
    def obs_loss(self):
        """Per-row sum of e^2/2 (the optimal-brain-surgeon increments)."""
        return 0.5 * np.sum(self.err * self.err, axis=1)


def _check_group(d, group, block):
    if group < 0:
        raise ValueError("group must be >= 0")
    if group and d % group:
        raise ValueError("group must divide d")


def gptq_quantize(w, u, bits: int, grid: str = GRID_ASYM, group: int = 0,
                  block: int = 128, follow_codes=None, follow_zeros=None,
                  band: float = 1e-3, blocked: bool = True,
                  col_grid=None) -> QuantResult:
    """Quantize W [m, d] column by column in natural order with the factor U.

    [FDE] figure "Quantize a column, correct the rest", steps 1-4, for column i:
      1. round w_i to the grid, giving q_i;
      2. err = (w_i - q_i) / U_ii with U = chol(H^-1);
      3. W[:, i+1:] -= err x U[i, i+1:];
      4. the updates are applied in blocks of 128 columns.
    [FDE] section 01: one fixed column order for every row; updates batched
    in blocks of 128 so the GPU is not waiting on memory.
    [NUB] "Proposed method": lazy batch updates.

    blocked=True applies step 3 inside a block immediately and to the columns
    after the block once, at the block's end (W[:, end:] -= E_blk U[blk, end:]);
    blocked=False applies step 3 to all later columns at every column. Both
    give the same result in exact arithmetic. A group grid is fitted at the
    group's first column j on the current weights, i.e. with every update of
    the columns before j applied: where the group reaches past the block, the
    block's updates of columns b0 .. j-1, which the blocked form applies only
    at the block's end, are added for the fit (W[:, end:j+g] - E[:, b0:j]
    U[b0:j, end:j+g]).

    follow_codes (optional, [m, d]): the codes of another implementation. At
    every element the oracle computes its own pre-round value p and code; a
    differing code is a band mismatch when it is an adjacent code and p lies
    within `band` grid units of the boundary between the two, else a hard
    mismatch. In both cases the oracle then continues with the given code, so
    that one legitimate choice at a boundary does not cascade down the row.
    follow_zeros does the same for the integer zero points ([m, ngroups]; for
    one grid per row [m, 1]), see follow_zero_points.

    col_grid (optional, (s [m, d], z [m, d])): a fixed grid for every column,
    fitted beforehand (static groups); no grid is fitted in the loop, and
    res.scales / res.zeros are left to the caller.
    """
    w = np.array(w, dtype=np.float64, copy=True)
    u = np.asarray(u, dtype=np.float64)
    m, d = w.shape
    if u.shape != (d, d):
        raise ValueError("U must be [d, d]")
    _check_group(d, group, block)
    ngroups = d // group if group else 1
    res = QuantResult(m, d, ngroups)
    maxq = maxq_of(bits, grid)

    if col_grid is not None:
        s_col = np.asarray(col_grid[0], dtype=np.float64)
        z_col = np.asarray(col_grid[1]).astype(np.int64)
        if s_col.shape != (m, d) or z_col.shape != (m, d):
            raise ValueError("col_grid must be two [m, d] arrays")
        group = 0
    elif group == 0:
        s, z, _ = fit_grid(w, bits, grid)
        if follow_zeros is not None and grid == GRID_ASYM:
            z, zb, zh = follow_zero_points(w, s, z, np.asarray(follow_zeros)[:, 0], band)
            res.zero_band_mismatch += zb
            res.zero_hard_mismatch += zh
        res.scales[:, 0] = s
        res.zeros[:, 0] = z
    step = block if blocked else d
    for b0 in range(0, d, step):
        b1 = min(b0 + step, d)
        for j in range(b0, b1):
            if group and j % group == 0:
                cur = w[:, j:j + group]
                if j + group > b1 and j > b0:
                    # the part past the block still lacks this block's updates of columns b0 .. j-1
                    cur = cur.copy()
                    cur[:, b1 - j:] -= res.err[:, b0:j] @ u[b0:j, b1:j + group]
                s, z, _ = fit_grid(cur, bits, grid)
                if follow_zeros is not None and grid == GRID_ASYM:
                    z, zb, zh = follow_zero_points(cur, s, z,
                                                   np.asarray(follow_zeros)[:, j // group], band)
                    res.zero_band_mismatch += zb
                    res.zero_hard_mismatch += zh
                res.scales[:, j // group] = s
                res.zeros[:, j // group] = z
            if col_grid is not None:
                s, z = s_col[:, j], z_col[:, j]
            col = w[:, j]
            p = col / s + z
            c = np.clip(np.rint(p), 0, maxq).astype(np.int64)
            res.p[:, j] = p
            res.dist[:, j] = boundary_distance(p, maxq)
            if follow_codes is not None:
                fc = np.asarray(follow_codes)[:, j].astype(np.int64)
                diff = fc != c
                if np.any(diff):
                    lowc = np.minimum(fc, c)
                    near = np.abs(p - (lowc + 0.5)) < band
                    adj = np.abs(fc - c) == 1
                    ok = diff & near & adj
                    bad = diff & ~(near & adj)
                    res.band_mismatch += int(np.sum(ok))
                    nbad = int(np.sum(bad))
                    if nbad:
                        res.hard_mismatch += nbad
                        for r in np.nonzero(bad)[0][:16]:
                            res.hard_positions.append((int(r), j))
                    c = fc
            q = s * (c - z)
            e = (col - q) / u[j, j]
            res.codes[:, j] = c
            res.w_hat[:, j] = q
            res.err[:, j] = e
            if blocked:
                w[:, j + 1:b1] -= np.outer(e, u[j, j + 1:b1])
            else:
                w[:, j + 1:] -= np.outer(e, u[j, j + 1:])
        if blocked and b1 < d:
            w[:, b1:] -= res.err[:, b0:b1] @ u[b0:b1, b1:]
    return res


def rtn_quantize(w, bits: int, grid: str = GRID_ASYM, group: int = 0) -> QuantResult:
    """Round-to-nearest on the same grid: the fit on the original weights
    (per row, or per group of original values), no error feedback.

    [FDE] "The paper in one minute": rounding each weight to the nearest grid
    value works at 8 bits and fails at 3-4 bits on large models; it is the
    baseline GPTQ is measured against (Table 3 in the figure).
    """
    w = np.asarray(w, dtype=np.float64)
    m, d = w.shape
    ngroups = d // group if group else 1
    res = QuantResult(m, d, ngroups)
    maxq = maxq_of(bits, grid)
    width = group if group else d
    for g0 in range(0, d, width):
        v = w[:, g0:g0 + width]
        s, z, _ = fit_grid(v, bits, grid)
        p = v / s[:, None] + z[:, None]
        c = np.clip(np.rint(p), 0, maxq).astype(np.int64)
        res.codes[:, g0:g0 + width] = c
        res.w_hat[:, g0:g0 + width] = s[:, None] * (c - z[:, None])
        res.p[:, g0:g0 + width] = p
        res.dist[:, g0:g0 + width] = boundary_distance(p, maxq)
        res.scales[:, g0 // width] = s
        res.zeros[:, g0 // width] = z
    return res


def quantize_layer(w, x_chunks, bits: int, grid: str = GRID_ASYM, group: int = 0,
                   block: int = 128, percdamp: float = 0.01, **kw):
    """The whole hot path on one layer: H, damping, U, column loop.

    Returns (result, H, U, lambda)."""
    h = hessian(x_chunks)
    hd, lam = damp(h, percdamp)
    u = inverse_hessian_factor(hd)
    res = gptq_quantize(w, u, bits, grid, group, block, **kw)
    return res, h, u, lam


# ---------------------------------------------------------------------------
# Act-order (desc_act) and static groups. The pages name both options and
# nothing more: [ZLY] "实践指南" passes desc_act (sort the columns by their
# activations, off by default) and "超参数选择" lists its default; [CSDN] lists
# --desc_act and --static_groups among the tool's parameters. Readings:
#  * the size of column j's activations is H_jj = 2 sum_t x_tj^2, and the
#    columns are quantized in descending H_jj, ties in index order;
#  * without static groups, groups are runs of g consecutive columns in that
#    order, each fitted at its first column on the current (updated) weights;
#  * with static groups, the grid of every natural group of g columns is
#    fitted before the loop on the original weights, and each column keeps its
#    natural group's grid wherever the order puts it.
# ---------------------------------------------------------------------------
def act_order_perm(h) -> np.ndarray:
    """perm[j] = the natural column quantized j-th: descending diag(H), ties in
    index order."""
    dg = np.diag(np.asarray(h, dtype=np.float64))
    return np.argsort(-dg, kind="stable")


def static_group_grids(w, bits: int, grid: str, group: int):
    """Grid of every natural group of `group` columns, fitted on the original
    weights: (s [m, d/group], z [m, d/group])."""
    w = np.asarray(w, dtype=np.float64)
    m, d = w.shape
    ng = d // group
    s = np.zeros((m, ng))
    z = np.zeros((m, ng), dtype=np.int64)
    for k in range(ng):
        s[:, k], z[:, k], _ = fit_grid(w[:, k * group:(k + 1) * group], bits, grid)
    return s, z


def gptq_quantize_ordered(w, u_perm, perm, bits: int, grid: str = GRID_ASYM, group: int = 0,
                          static_groups: bool = False, block: int = 128, follow_codes=None,
                          follow_zeros=None, band: float = 1e-3, blocked: bool = True):
    """The column loop in the order perm, with U the factor of the permuted
    damped Hessian (H_d[perm][:, perm]). Inputs and outputs are in natural
    column order.

    Returns (res, g_idx): res.codes / w_hat / err / p / dist at natural
    columns; res.scales / res.zeros [m, ngroups] by group number; g_idx [d] the
    group number of every natural column (0 for one grid per row).
    follow_codes / follow_zeros are in natural order like the outputs."""
    w = np.asarray(w, dtype=np.float64)
    perm = np.asarray(perm, dtype=np.int64)
    m, d = w.shape
    if sorted(perm.tolist()) != list(range(d)):
        raise ValueError("perm is not a permutation of the columns")
    _check_group(d, group, block)
    wp = w[:, perm]
    fc = None if follow_codes is None else np.asarray(follow_codes)[:, perm]
    if group and static_groups:
        s_g, z_g = static_group_grids(w, bits, grid, group)
        zb = zh = 0
        if follow_zeros is not None and grid == GRID_ASYM:
            # the zero points of another implementation, judged as in the loop:
            # an adjacent zero is taken when -lo/s lies within `band` of the
            # half-integer between the two (an exact tie such as a group whose
            # extremes are +-a, where -lo/s = maxq/2, falls either way in
            # finite precision); anything else is a hard mismatch
            fz = np.asarray(follow_zeros).astype(np.int64)
            for k in range(d // group):
                z_g[:, k], b_k, h_k = follow_zero_points(w[:, k * group:(k + 1) * group], s_g[:, k], z_g[:, k],
                                                         fz[:, k], band)
                zb += b_k
                zh += h_k
        gcol = perm // group  # natural group of the j-th quantized column
        res_p = gptq_quantize(wp, u_perm, bits, grid, 0, block, follow_codes=fc, band=band,
                              blocked=blocked, col_grid=(s_g[:, gcol], z_g[:, gcol]))
        res = QuantResult(m, d, d // group)
        res.scales[:] = s_g
        res.zeros[:] = z_g
        res.zero_band_mismatch, res.zero_hard_mismatch = zb, zh
        g_idx = np.arange(d) // group
    else:
        res_p = gptq_quantize(wp, u_perm, bits, grid, group, block, follow_codes=fc,
                              follow_zeros=follow_zeros, band=band, blocked=blocked)
        res = QuantResult(m, d, res_p.scales.shape[1])
        res.scales[:] = res_p.scales
        res.zeros[:] = res_p.zeros
        res.zero_band_mismatch = res_p.zero_band_mismatch
        res.zero_hard_mismatch = res_p.zero_hard_mismatch
        g_idx = np.zeros(d, dtype=np.int64)
        if group:
            g_idx[perm] = np.arange(d) // group
    for name in ("codes", "w_hat", "err", "p", "dist"):
        getattr(res, name)[:, perm] = getattr(res_p, name)
    res.band_mismatch = res_p.band_mismatch
    res.hard_mismatch = res_p.hard_mismatch
    res.hard_positions = [(r, int(perm[j])) for r, j in res_p.hard_positions]
    return res, g_idx


def quantize_layer_act_order(w, x_chunks, bits: int, grid: str = GRID_ASYM, group: int = 0,
                             static_groups: bool = False, block: int = 128,
                             percdamp: float = 0.01, **kw):
    """The hot path with act-order: H, the order, the permuted damped H, its
    factor, the column loop in that order.

    Returns (result, g_idx, perm, H, U_perm, lambda); H is in natural order."""
    h = hessian(x_chunks)
    perm = act_order_perm(h)
    hd, lam = damp(h[np.ix_(perm, perm)], percdamp)
    u = inverse_hessian_factor(hd)
    res, g_idx = gptq_quantize_ordered(w, u, perm, bits, grid, group, static_groups, block, **kw)
    return res, g_idx, perm, h, u, lam


# ---------------------------------------------------------------------------
# Packing of the integer codes.
# ---------------------------------------------------------------------------
def pack_codes(codes, bits: int) -> np.ndarray:
    """Row-wise LSB-first bitstream: code j of a row occupies bits
    [j*b, (j+1)*b) of the row's stream; bit t of the stream is bit (t mod 32)
    of word t // 32. A code that straddles two words is split, low bits first.

    [FDE] section 01 and the figure: the output is 3-bit (or 4-bit) weights
    that an inference kernel reads and dequantizes on the fly. The pages do not
    fix a layout; this is the stated reading. d*b must be a multiple of 32.
    """
    codes = np.asarray(codes, dtype=np.int64)
    m, d = codes.shape
    if (d * bits) % 32:
        raise ValueError("d*bits must be a multiple of 32")
    nwords = d * bits // 32
    out = np.zeros((m, nwords), dtype=np.uint64)
    for j in range(d):
        c = codes[:, j].astype(np.uint64)
        for t in range(bits):
            pos = j * bits + t
            bit = (c >> np.uint64(t)) & np.uint64(1)
            out[:, pos // 32] |= bit << np.uint64(pos % 32)
    return out.astype(np.uint32)


def unpack_codes(words, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_codes."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    m = words.shape[0]
    codes = np.zeros((m, d), dtype=np.int64)
    for j in range(d):
        v = np.zeros(m, dtype=np.uint64)
        for t in range(bits):
            pos = j * bits + t
            bit = (words[:, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)
            v |= bit << np.uint64(t)
        codes[:, j] = v.astype(np.int64)
    return codes


# ---------------------------------------------------------------------------
# Generation with the packed weights. [FDE] section 01: the 3/4-bit weights are
# read by an inference kernel that dequantizes them on the fly; [NUB] "Key
# findings": end-to-end speedups of 3-bit OPT-175B generation (about 3.25x on
# A100, 4.5x on A6000) over fp16. One token (batch 1) is a matrix-vector
# product with every layer's dequantized weights.
# ---------------------------------------------------------------------------
def dequant_matvec(words, scales, zeros, bits: int, group: int, x, g_idx=None) -> np.ndarray:
    """y[r] = sum_j s[r, g(j)] (c[r, j] - z[r, g(j)]) x[j] in fp64, with c the
    codes unpacked from the row bitstreams and g(j) = j // group (0 for one grid
    per row), or g(j) = g_idx[j] when a group index is given (act-order
    without static groups, where the k-th group is the k-th run of columns in
    the quantization order). The product of W_hat = s (c - z) with x."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[0]
    c = unpack_codes(words, bits, d)
    if g_idx is not None:
        gidx = np.asarray(g_idx, dtype=np.int64)
    else:
        gidx = np.arange(d) // group if group else np.zeros(d, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float64)[:, gidx]
    z = np.asarray(zeros).astype(np.int64)[:, gidx]
    return (s * (c - z)) @ x
