"""Full-size layers through the C ABI, in the launch configuration the
benchmark times (one gptq_accumulate_hessian call over all 262144 tokens, fp64
H; the R factor for the OPT-175B layers, fp64 U for the OPT-13B one).

* OPT-13B attention projection (5120 x 5120, 262144 tokens, 3-bit g128): the
  whole oracle runs on every row, and the usual parity gates apply.
* OPT-175B q (12288 x 12288), fc1 (49152 x 12288, 3-bit g128) and the extreme
  regime on the fc1 shape (2-bit and ternary g128, one W and one X): the GPU
  quantizes the whole layer from R, the Cholesky factor of H_d (the benchmark's
  path); the oracle builds its own fp64 H from all 262144
  tokens, damps it and factors it, then runs follow mode and a free run on
  258 sampled rows (rows are independent given U, and every grid is fitted
  within its row). The usual gates apply to those rows.
* OPT-175B fc2 (12288 x 49152): the oracle's own H over all 262144 tokens
  would cost 1.3e15 fp64 flops on the host, about half an hour on 16 cores,
  more than a test may take. Code parity there runs on a token-count stand-in:
  the whole layer on the GPU at its full width, calibrated on the first 16384
  of its tokens (fewer tokens than features, so H is singular before damping:
  a harder case for the factor's accuracy than the full token count), against
  the oracle's own H over those tokens, its factor and follow mode on 258
  sampled rows, with every gate. The full token count has the checks on
  sampled outputs the oracle computes one by one, and on properties that hold
  at any size:
  - sampled entries of H against the oracle's fp64 Hessian of those columns;
  - lambda against damp * mean(diag H) (diag in fp64 from X);
  - U upper with a positive diagonal, and U^T U H_d e_j = e_j on sampled
    columns, with H_d = H + lambda I from the GPU's H (fp64 U and products);
  - W_hat = s * (code - z) exactly, codes within the grid, packing bit-exact
    (the oracle's packer on the unpacked codes), on sampled rows;
  - on sampled rows: the OBS loss identity sum_j e_j^2 / 2 = ||(w - w_hat) X^T||^2
    + lambda / 2 ||w - w_hat||^2 for the GPU's own trajectory, and the GPTQ loss
    below the oracle's round-to-nearest loss on the same grid.
"""

from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle as O
from post_weight_quantization_18_amd import gptq as G
from post_weight_quantization_18_amd import synthetic as S

from parity_util import (assert_gates, compare_layer, compare_rows, device_factor_r, gpu_layer, oracle_factor,
                         rows_of, sample_rows, say)

pytestmark = pytest.mark.gpu

CHUNK = 262144
DEV = torch.device("cuda:0")


@pytest.mark.timeout(1200)
def test_layer_parity_opt13b_attn_full():
    cfg = S.CONFIGS["opt13b-attn"]
    say(f"[case] full layer {cfg.name} m={cfg.m} d={cfg.d} n={cfg.n_tokens}")
    w, x = S.make_layer(cfg, device="cuda")
    w, x = w.cpu(), x.cpu()
    gpu = gpu_layer(w, x, cfg.bits, cfg.group, cfg.grid, cfg.damp, chunk_tokens=CHUNK)
    assert_gates(compare_layer(w, x, cfg.bits, cfg.group, cfg.grid, gpu, cfg.damp, cfg.name))


_CODE_PARITY = [("opt175b-q", ["opt175b-q"]), ("opt175b-fc1", ["opt175b-fc1"]),
                ("opt175b-fc1-extreme", ["opt175b-fc1-2bit", "opt175b-fc1-ternary"])]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("label,names", _CODE_PARITY, ids=[c[0] for c in _CODE_PARITY])
def test_code_parity_full_size_sampled_rows(label, names):
    """The whole layer on the GPU; the oracle's own H, lambda and U from all
    262144 tokens; follow mode on 258 sampled rows with every gate."""
    cfgs = [S.CONFIGS[n] for n in names]
    c0 = cfgs[0]
    assert all((c.m, c.d, c.n_tokens, c.config_id, c.layer_id) == (c0.m, c0.d, c0.n_tokens, c0.config_id,
                                                                      c0.layer_id) for c in cfgs)
    say(f"[case] full-size code parity {label} m={c0.m} d={c0.d} n={c0.n_tokens} grids="
        f"{[(c.bits, c.grid, c.group) for c in cfgs]}")
    t0 = time.time()
    w = S.make_weights(c0, DEV)
    x = S.make_activations(c0, DEV)
    H, U, lam = device_factor_r(c0.d, x, c0.damp)
    rows = sample_rows(c0.m, 21)
    gpu_rows = []
    for c in cfgs:
        res = G.quantize_layer(w, U, c.bits, c.group, c.grid, factor="R")
        torch.cuda.synchronize()
        gpu_rows.append(rows_of(res, rows, c.bits, c.d))
        del res
    factor = {"H": H.cpu().numpy(), "U": U.cpu().double().numpy(), "lam": lam, "u_eps": 2.0 ** -53, "factor": "R"}
    wn = w[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    xh = x.cpu().numpy()
    del H, U, x
    torch.cuda.empty_cache()
    say(f"[step] {label}: GPU layer(s) done in {time.time() - t0:.1f} s; oracle H over {xh.shape[0]} tokens")
    t1 = time.time()
    h, lam_o, u, hd = oracle_factor(xh, c0.damp)
    del xh
    say(f"[step] {label}: oracle H, lambda, U in {time.time() - t1:.1f} s")
    for c, gr in zip(cfgs, gpu_rows):
        gr.update(factor)
        stats = compare_rows(wn, gr, h, lam_o, u, hd, c.bits, c.group, c.grid, f"{c.name} ({len(rows)} rows)")
        assert_gates(stats)


FC2_STAND_IN_TOKENS = 16384


@pytest.mark.timeout(1200)
def test_code_parity_fc2_full_width_token_stand_in():
    """OPT-175B fc2 at its full width (12288 x 49152) on the first 16384 of its
    262144 tokens: the GPU's H, R and whole layer in the benchmark's path; the
    oracle's H over the same tokens chunk by chunk, lambda, its R and U = R^-1,
    then follow mode and a free run on 258 sampled rows; every gate."""
    from block_parity_harness import compare_rows_in_steps, oracle_factor_in_steps

    cfg = S.CONFIGS["opt175b-fc2"]
    n = FC2_STAND_IN_TOKENS
    say(f"[case] fc2 full-width code parity m={cfg.m} d={cfg.d} on the first {n} of {cfg.n_tokens} tokens")
    t0 = time.time()
    w = S.make_weights(cfg, DEV)
    x = S.make_activations(cfg, DEV)[:n].contiguous()
    torch.cuda.empty_cache()
    H, R, lam = device_factor_r(cfg.d, x, cfg.damp)
    res = G.quantize_layer(w, R, cfg.bits, cfg.group, cfg.grid, factor="R")
    torch.cuda.synchronize()
    rows = sample_rows(cfg.m, 21 + cfg.layer_id)
    gr = rows_of(res, rows, cfg.bits, cfg.d)
    gr.update({"H": H.cpu().numpy(), "U": R.cpu().numpy(), "lam": lam, "u_eps": 2.0 ** -53, "factor": "R"})
    wn = w[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    xh = x.cpu().numpy()
    del H, R, x, w, res
    torch.cuda.empty_cache()
    say(f"[step] fc2 stand-in: GPU layer done in {time.time() - t0:.1f} s; oracle H over {n} tokens")
    oracle = oracle_factor_in_steps(xh, cfg.damp, log=say)
    del xh
    stats = compare_rows_in_steps(wn, gr, oracle, cfg.bits, cfg.group, cfg.grid,
                                  f"{cfg.name} first {n} tokens ({len(rows)} rows)", log=say)
    say(f"[parity] fc2 stand-in: hard={stats['hard']} identical={stats['identical']:.7f} "
        f"scale_rel={stats['scale_rel']:.3e} u_rel={stats['u_rel']:.3e} h_rel={stats['h_rel']:.3e}")
    assert_gates(stats)


def _run_full(cfg):
    """The three entry points on cuda:0 with device-resident results (U fp64)."""
    w = S.make_weights(cfg, DEV)
    x = S.make_activations(cfg, DEV)
    d = cfg.d
    H = torch.empty(d, d, dtype=torch.float64, device=DEV)
    for i, t0 in enumerate(range(0, cfg.n_tokens, CHUNK)):
        G.accumulate_hessian(H, x[t0:t0 + CHUNK], accumulate=i > 0)
    U, info, lam = G.prepare_hinv(H, cfg.damp, u_dtype=torch.float64)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    res = G.quantize_layer(w, U, cfg.bits, cfg.group, cfg.grid)
    torch.cuda.synchronize()
    return w, x, H, U, float(lam.item()), res


def _sampled_h(x, H, rng, k=48):
    d = H.shape[0]
    cols = np.unique(np.concatenate([rng.choice(d, k, replace=False), [0, d - 1]]))
    xs = x[:, torch.as_tensor(cols, device=DEV)].cpu().numpy()
    h_orc = O.hessian([xs[i:i + 65536] for i in range(0, xs.shape[0], 65536)])
    h_gpu = H[torch.as_tensor(cols, device=DEV)][:, torch.as_tensor(cols, device=DEV)].cpu().numpy()
    il = np.tril_indices(len(cols))
    scale = np.sqrt(np.outer(np.diag(h_orc), np.diag(h_orc)))[il]
    return float(np.max(np.abs(h_gpu[il] - h_orc[il]) / scale))


def _diag_h(x):
    acc = torch.zeros(x.shape[1], dtype=torch.float64, device=DEV)
    for t0 in range(0, x.shape[0], 4096):
        xc = x[t0:t0 + 4096].double()
        acc += (xc * xc).sum(0)
    return 2.0 * acc


def _hd_column(H, j, lam):
    """Column j of H_d = H + lambda I from the GPU's own H (lower triangle valid):
    U is checked against the matrix it factors, so that H's own rounding,
    amplified by the condition number, does not enter this check."""
    v = torch.cat([H[j, :j], H[j:, j]]).clone()
    v[j] += lam
    return v


def _row_losses(x, delta):
    """||delta_r X^T||^2 per row, fp64 over token chunks."""
    out = torch.zeros(delta.shape[0], dtype=torch.float64, device=DEV)
    for t0 in range(0, x.shape[0], 4096):
        y = delta @ x[t0:t0 + 4096].double().t()
        out += (y * y).sum(1)
    return out


_FULL = ["opt175b-fc2"]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", _FULL)
def test_layer_properties_full_size(name):
    cfg = S.CONFIGS[name]
    say(f"[case] full-size properties {name} m={cfg.m} d={cfg.d} n={cfg.n_tokens} bits={cfg.bits} "
        f"grid={cfg.grid} group={cfg.group}")
    rng = np.random.default_rng(11)
    w, x, H, U, lam, res = _run_full(cfg)
    d, m = cfg.d, cfg.m

    h_err = _sampled_h(x, H, rng)
    say(f"[check] {name}: sampled H max |dH_ij| / sqrt(H_ii H_jj) = {h_err:.2e}")
    assert h_err <= 1e-6

    diag = _diag_h(x)
    lam_ref = cfg.damp * float(diag.mean().item())
    say(f"[check] {name}: lambda rel err {abs(lam - lam_ref) / lam_ref:.2e}")
    assert abs(lam - lam_ref) <= 1e-6 * lam_ref  # lambda inherits H's ~1e-8 relative rounding

    du = torch.diagonal(U)
    assert bool((du > 0).all())
    some_rows = torch.as_tensor(rng.choice(d, 8, replace=False), device=DEV)
    for i in some_rows.tolist():
        assert bool((U[i, :i] == 0).all())
    worst = 0.0
    for j in rng.choice(d, 3, replace=False).tolist():
        v = _hd_column(H, j, lam)
        y = U.t() @ (U @ v)
        e = torch.zeros_like(y)
        e[j] = 1.0
        worst = max(worst, float((y - e).abs().max().item()))
    say(f"[check] {name}: max |U^T U H_d e_j - e_j| = {worst:.2e}")
    assert worst <= 1e-6

    rows = np.sort(rng.choice(m, 24, replace=False))
    rt = torch.as_tensor(rows, device=DEV)
    codes = O.unpack_codes(res["qcodes"][rt].cpu().numpy().view(np.uint32), cfg.bits, d)
    maxq = O.maxq_of(cfg.bits, cfg.grid)
    assert codes.max() <= maxq
    scales = res["scales"][rt].cpu().numpy()
    zeros = res["zeros"][rt].cpu().numpy().astype(np.int64)
    assert zeros.max() <= maxq
    gidx = (np.arange(d) // cfg.group) if cfg.group else np.zeros(d, np.int64)
    w_hat = res["w_hat"][rt].cpu().numpy()
    expect = scales[:, gidx].astype(np.float32) * (codes.astype(np.float32) - zeros[:, gidx].astype(np.float32))
    assert np.array_equal(w_hat, expect)
    assert np.array_equal(res["qcodes"][rt].cpu().numpy().view(np.uint32), O.pack_codes(codes, cfg.bits))

    wr = w[rt].double()
    delta = wr - res["w_hat"][rt].double()
    loss = _row_losses(x, delta)
    obs = res["err_sq"][rt].double()
    ident = loss + 0.5 * lam * (delta * delta).sum(1)
    obs_rel = float(((obs - ident).abs() / ident).max().item())
    rtn = O.rtn_quantize(wr.cpu().numpy(), cfg.bits, cfg.grid, cfg.group)
    loss_rtn = _row_losses(x, wr - torch.as_tensor(rtn.w_hat, device=DEV))
    ratio = float(loss.sum().item() / loss_rtn.sum().item())
    say(f"[check] {name}: OBS identity max rel err {obs_rel:.2e}; GPTQ / RTN loss on {len(rows)} rows = {ratio:.4f}")
    assert obs_rel <= 1e-3
    assert ratio < 1.0


# ---------------------------------------------------------------------------
# act-order (desc_act) at full size
# ---------------------------------------------------------------------------
@pytest.mark.timeout(1200)
def test_act_order_parity_opt13b_attn_full():
    """The whole oracle's act-order path at 5120 x 5120, 262144 tokens."""
    from parity_util import assert_ordered_gates, compare_layer_ordered, gpu_layer_ordered
    cfg = S.CONFIGS["opt13b-attn"]
    say(f"[case] full layer act-order {cfg.name} m={cfg.m} d={cfg.d} n={cfg.n_tokens}")
    w, x = S.make_layer(cfg, device="cuda")
    w, x = w.cpu(), x.cpu()
    gpu = gpu_layer_ordered(w, x, cfg.bits, cfg.group, cfg.grid, False, cfg.damp)
    stats = compare_layer_ordered(w, x, cfg.bits, cfg.group, cfg.grid, False, gpu, cfg.damp, cfg.name + "-act-order")
    assert_ordered_gates(stats, False, cfg.group)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,static", [("opt175b-q", True)])
def test_act_order_properties_full_size(name, static):
    """d = 12288 with act-order: the order against the oracle's on the GPU's
    own diagonal and against H_jj from X, sampled entries of the permuted H,
    U against the permuted H_d, and the output checks of the natural-order
    test with g_idx."""
    cfg = S.CONFIGS[name]
    say(f"[case] full-size act-order properties {name} static={static} m={cfg.m} d={cfg.d}")
    rng = np.random.default_rng(12)
    w = S.make_weights(cfg, DEV)
    x = S.make_activations(cfg, DEV)
    d, m = cfg.d, cfg.m
    H = torch.empty(d, d, dtype=torch.float64, device=DEV)
    G.accumulate_hessian(H, x, accumulate=False)
    perm = G.act_order(H)
    Hp = G.permute_hessian(H, perm)
    U, info, lam_t = G.prepare_hinv(Hp, cfg.damp, u_dtype=torch.float64)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    lam = float(lam_t.item())
    res = G.quantize_layer_ordered(w, U, perm, cfg.bits, cfg.group, cfg.grid, static)
    torch.cuda.synchronize()

    p = perm.cpu().numpy().astype(np.int64)
    hdiag = torch.diagonal(H).cpu().numpy()
    np.testing.assert_array_equal(p, O.act_order_perm(np.diag(hdiag)))
    dx = _diag_h(x).cpu().numpy()[p]
    assert np.all(dx[1:] <= dx[:-1] * (1 + 1e-7))
    say(f"[check] {name}: order bit-exact on the GPU's diagonal; H_jj from X non-increasing along it")

    ii = np.sort(rng.choice(d, 64, replace=False))
    pt = torch.as_tensor(p, device=DEV)
    for i in ii.tolist():
        jj = torch.arange(0, i + 1, max(1, i // 50), device=DEV)
        a = torch.maximum(pt[i], pt[jj])
        b = torch.minimum(pt[i], pt[jj])
        assert torch.equal(Hp[i, jj], H[a, b])
    worst = 0.0
    for j in rng.choice(d, 3, replace=False).tolist():
        v = _hd_column(Hp, j, lam)
        y = U.t() @ (U @ v)
        e = torch.zeros_like(y)
        e[j] = 1.0
        worst = max(worst, float((y - e).abs().max().item()))
    say(f"[check] {name}: sampled Hp exact; max |U^T U Hp_d e_j - e_j| = {worst:.2e}")
    assert worst <= 1e-6

    gidx = res["g_idx"].cpu().numpy().astype(np.int64)
    if static:
        np.testing.assert_array_equal(gidx, np.arange(d) // cfg.group)
    else:
        want = np.empty(d, np.int64)
        want[p] = np.arange(d) // cfg.group
        np.testing.assert_array_equal(gidx, want)
    rows = np.sort(rng.choice(m, 24, replace=False))
    rt = torch.as_tensor(rows, device=DEV)
    codes = O.unpack_codes(res["qcodes"][rt].cpu().numpy().view(np.uint32), cfg.bits, d)
    maxq = O.maxq_of(cfg.bits, cfg.grid)
    assert codes.max() <= maxq
    scales = res["scales"][rt].cpu().numpy()
    zeros = res["zeros"][rt].cpu().numpy().astype(np.int64)
    w_hat = res["w_hat"][rt].cpu().numpy()
    expect = scales[:, gidx].astype(np.float32) * (codes.astype(np.float32) - zeros[:, gidx].astype(np.float32))
    assert np.array_equal(w_hat, expect)
    wr = w[rt].double()
    if static:
        s_o, z_o = O.static_group_grids(wr.cpu().numpy(), cfg.bits, cfg.grid, cfg.group)
        assert float(np.max(np.abs(scales - s_o) / s_o)) <= 1e-6
        assert int(np.max(np.abs(zeros - z_o))) <= 1
    delta = wr - res["w_hat"][rt].double()
    loss = _row_losses(x, delta)
    obs = res["err_sq"][rt].double()
    ident = loss + 0.5 * lam * (delta * delta).sum(1)
    obs_rel = float(((obs - ident).abs() / ident).max().item())
    rtn = O.rtn_quantize(wr.cpu().numpy(), cfg.bits, cfg.grid, cfg.group)
    loss_rtn = _row_losses(x, wr - torch.as_tensor(rtn.w_hat, device=DEV))
    ratio = float(loss.sum().item() / loss_rtn.sum().item())
    say(f"[check] {name}: OBS identity max rel err {obs_rel:.2e}; act-order / RTN loss on {len(rows)} rows = {ratio:.4f}")
    assert obs_rel <= 1e-3
    assert ratio < 1.0
