"""Resume logic of the block harness (host only): a layer counts as done when
its results line and its output file exist; q, k and v share one input, so
their group runs while any of its requested layers is missing."""

import json
import os

import block_parity_harness as BH


def _done(tmp_path, layers, with_npz=True):
    with open(tmp_path / "results.jsonl", "w") as fh:
        for l in layers:
            fh.write(json.dumps({"config": BH.BLOCK, "layer": l}) + "\n")
            if with_npz:
                (tmp_path / f"{l}.npz").write_bytes(b"")


def test_fresh_run_plans_every_group():
    todo = BH.plan(list(BH.LAYERS), set())
    assert [w for _, w in todo] == [["q", "k", "v"], ["out"], ["fc1"], ["fc2"]]


def test_resume_continues_at_the_next_layer(tmp_path):
    _done(tmp_path, ["q", "k", "v", "out"])
    done = BH.completed(str(tmp_path))
    assert done == {"q", "k", "v", "out"}
    assert [w for _, w in BH.plan(list(BH.LAYERS), done)] == [["fc1"], ["fc2"]]


def test_a_layer_without_its_outputs_is_not_done(tmp_path):
    _done(tmp_path, ["q", "k"], with_npz=False)
    (tmp_path / "q.npz").write_bytes(b"")
    done = BH.completed(str(tmp_path))
    assert done == {"q"}
    todo = BH.plan(list(BH.LAYERS), done)
    assert todo[0] == (["q", "k", "v"], ["k", "v"])


def test_layer_work_counts():
    flops, nbytes = BH.layer_work(BH.S.CONFIGS["opt175b-fc2"])
    m, d, n = 12288, 49152, 262144
    assert flops["syrk"] == n * d * (d + 1) and flops["chain"] == d ** 3 / 3
    assert nbytes["x"] == 2 * n * d and nbytes["outputs"] == m * d * 3 // 8 + m * (d // 128) * 5 + 4 * m


def test_stepwise_oracle_factor_matches_the_oracle():
    """The harness's stepwise oracle factor (H chunk by chunk, U = R^-1 by column
    blocks) gives the oracle's H bit for bit and its U to fp64 rounding."""
    import numpy as np

    from parity_util import oracle_factor

    rng = np.random.default_rng(7)
    x = (rng.standard_normal((300, 96)) * np.linspace(0.3, 2.0, 96)).astype(np.float16)
    h1, lam1, u1, hd1 = oracle_factor(x, 0.01, chunk=128)
    h2, lam2, u2, hd2, r2 = BH.oracle_factor_in_steps(x, 0.01, chunk=128)
    assert np.array_equal(h1, h2) and lam1 == lam2 and np.array_equal(hd1, hd2)
    assert np.linalg.norm(u2 - u1) <= 1e-12 * np.linalg.norm(u1)
    assert np.allclose(r2 @ r2.T, hd2, rtol=1e-12, atol=1e-12 * np.abs(hd2).max())


def test_upper_inverse_by_halves():
    """upper_inverse (halves down to small leaves, ragged splits included)
    against numpy's general inverse, and upper triangular."""
    import numpy as np
    rng = np.random.default_rng(9)
    for n, leaf in ((300, 64), (129, 32), (64, 64), (7, 2)):
        r = np.triu(rng.standard_normal((n, n))) + np.diag(np.full(n, 4.0))
        u = BH.upper_inverse(r, leaf=leaf)
        assert np.all(np.tril(u, -1) == 0.0)
        np.testing.assert_allclose(u, np.linalg.inv(r), rtol=1e-9, atol=1e-12)


def test_lower_rel_fro_by_row_blocks():
    """The blockwise distance of the lower triangles equals the symmetric
    Frobenius distance written out on a small case (upper parts ignored)."""
    import numpy as np

    from parity_util import lower_rel_fro
    rng = np.random.default_rng(11)
    d = 37
    a, b = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    sym = lambda m: np.tril(m) + np.tril(m, -1).T  # noqa: E731
    want = np.linalg.norm(sym(a) - sym(b)) / np.linalg.norm(sym(b))
    for rows in (5, 16, 64):
        assert abs(lower_rel_fro(a, b, rows=rows) - want) <= 1e-13 * want
