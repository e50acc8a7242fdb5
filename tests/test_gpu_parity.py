"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every test prints the case it is about to run before touching the GPU.
"""

import numpy as np
import pytest
import torch

import oracle as O
from post_weight_quantization_18_amd import gptq as G
from post_weight_quantization_18_amd import synthetic as S

from parity_util import assert_gates, compare_layer, gpu_layer, lower_rel_fro, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _library():
    G.load_library()
    assert torch.cuda.is_available()


# ---------------------------------------------------------------------------
# packing kernel: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits,m,d", [(2, 37, 96), (3, 5, 96), (3, 64, 128), (4, 33, 64), (8, 3, 32)])
def test_pack_kernel_bit_exact(bits, m, d):
    say(f"[case] pack bits={bits} m={m} d={d}")
    rng = np.random.default_rng(bits * 100 + m)
    codes = rng.integers(0, 1 << bits, size=(m, d)).astype(np.uint8)
    out = G.pack_codes(torch.from_numpy(codes).to(DEV), bits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, O.pack_codes(codes, bits))


# ---------------------------------------------------------------------------
# Hessian
# ---------------------------------------------------------------------------
def _x(cfg):
    return S.make_activations(cfg)


@pytest.mark.parametrize("h_dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("chunk", [None, 1000])
def test_hessian_parity_toy(h_dtype, chunk):
    cfg = S.CONFIGS["toy768"]
    say(f"[case] hessian toy768 h_dtype={h_dtype} chunk={chunk}")
    x = _x(cfg)
    xd = x.to(DEV)
    d = cfg.d
    H = torch.full((d, d), 7.0, dtype=h_dtype, device=DEV)
    if chunk is None:
        G.accumulate_hessian(H, xd, accumulate=False)
    else:
        for i, t0 in enumerate(range(0, x.shape[0], chunk)):
            G.accumulate_hessian(H, xd[t0:t0 + chunk], accumulate=i > 0)
    torch.cuda.synchronize()
    hg = H.cpu().double().numpy()
    ho = O.hessian(x.numpy())
    rel = lower_rel_fro(hg, ho)
    say(f"  rel_fro={rel:.3e}")
    assert rel <= (1e-7 if h_dtype == torch.float64 else 1e-6)
    assert np.all(hg[np.triu_indices(d, 1)] == 7.0)   # strictly upper triangle untouched


# d = 2336 and 4192: a last I-block of 32 and of 96 features, an empty tile past
# d; 4192 has 306 tiles, so 50 go to the stream-K ranges. From d = 12288 the
# feature-major form (X^T in the workspace): d = 13024 has 51 I-blocks (the
# last band of the tile order holds 3, the last I-block 224 features; 2652
# tiles, 92 by stream-K), d = 16416 a last I-block of 32 features (4290 tiles,
# 194 by stream-K), 700 tokens padded to 704.
@pytest.mark.parametrize("n,d", [(3000, 96), (64, 320), (1, 32), (70000, 512), (5000, 2336), (1100, 4192),
                                 (900, 13024), (700, 16416)])
def test_hessian_parity_ragged(n, d):
    say(f"[case] hessian ragged n={n} d={d}")
    rng = np.random.default_rng(n + d)
    x = torch.from_numpy((rng.standard_normal((n, d)) * 2).astype(np.float16))
    H = torch.empty(d, d, dtype=torch.float64, device=DEV)
    G.accumulate_hessian(H, x.to(DEV), accumulate=False)
    torch.cuda.synchronize()
    hg = H.cpu().numpy()
    ho = O.hessian(x.numpy())
    rel = lower_rel_fro(hg, ho)
    # elementwise: the fp16 products are exact in fp32 and each 16-token MFMA
    # step rounds once; the W/16 steps between folds can lose at most W/16 fp32
    # roundings of the running |sum|, bounded by 2 sum_t |x_ti x_tj| (twice
    # that, for rounding inside the instruction); a missing or doubled tile is
    # off by |H_ij|, ~1/sqrt(n) of that sum, far above the bound. The library
    # states its fold window W per call: 1024 tokens from 262144, 512 from
    # 65536, 256 below.
    w_fold = 1024 if n >= 262144 else 512 if n >= 65536 else 256
    habs = O.hessian(np.abs(x.numpy()))
    il = np.tril_indices(d)
    excess = np.abs(hg[il] - ho[il]) - (w_fold // 8) * 2.0 ** -24 * habs[il]
    say(f"  rel_fro={rel:.3e} worst elementwise excess over the bound {excess.max():.3e}")
    assert np.all(excess <= 0.0)
    assert rel <= 5e-7


def test_hessian_accumulate_and_empty():
    say("[case] hessian accumulate semantics and n=0")
    d = 64
    rng = np.random.default_rng(5)
    x1 = torch.from_numpy(rng.standard_normal((100, d)).astype(np.float16))
    x2 = torch.from_numpy(rng.standard_normal((37, d)).astype(np.float16))
    H = torch.empty(d, d, dtype=torch.float64, device=DEV)
    G.accumulate_hessian(H, x1.to(DEV), accumulate=False)
    G.accumulate_hessian(H, x2.to(DEV), accumulate=True)
    G.accumulate_hessian(H, x2[:0].to(DEV), accumulate=True)      # no tokens: unchanged
    torch.cuda.synchronize()
    rel = lower_rel_fro(H.cpu().numpy(), O.hessian([x1.numpy(), x2.numpy()]))
    assert rel <= 1e-7
    G.accumulate_hessian(H, x2[:0].to(DEV), accumulate=False)     # no tokens, overwrite: zero
    torch.cuda.synchronize()
    assert np.all(np.tril(H.cpu().numpy()) == 0)


# ---------------------------------------------------------------------------
# inverse-Hessian factor
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,u_dtype", [(768, torch.float64), (768, torch.float32), (96, torch.float64),
                                       (200, torch.float64), (1000, torch.float64), (4160, torch.float64),
                                       (64, torch.float64), (40, torch.float64),
                                       # large enough for the 128-tile trailing updates, ragged at 128
                                       (8256, torch.float64), (2049, torch.float64)])
def test_chain_parity(d, u_dtype):
    say(f"[case] chain d={d} u_dtype={u_dtype}")
    rng = np.random.default_rng(d)
    a = rng.standard_normal((4 * d, d)) @ np.diag(1.0 / np.arange(1, d + 1)) @ np.linalg.qr(rng.standard_normal((d, d)))[0]
    h = 2 * a.T @ a
    Hd = torch.from_numpy(h).to(DEV)
    U, info, lam = G.prepare_hinv(Hd, 0.01, u_dtype=u_dtype)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    hd_o, lam_o = O.damp(h, 0.01)
    uo = O.inverse_hessian_factor(hd_o)
    ug = U.cpu().double().numpy()
    rel = np.linalg.norm(ug - uo) / np.linalg.norm(uo)
    say(f"  U rel={rel:.3e} lam_rel={abs(float(lam.item()) - lam_o) / lam_o:.2e}")
    assert np.all(np.tril(ug, -1) == 0)
    assert rel <= (1e-10 if u_dtype == torch.float64 else 2e-7)
    assert abs(float(lam.item()) - lam_o) <= 1e-12 * lam_o


def test_hchol_parity_wide_tiles():
    """At d = 16960 the first trailing update (16448 wide) runs on 128 x 128
    tiles, the next ones on 128 x 64 down to 4096, then 64 x 64; ragged at 128.
    H = 2 A^T A + diag(c) from a 1024-token A keeps the host's oracle cheap."""
    d = 16960
    say(f"[case] hchol wide tiles d={d}")
    rng = np.random.default_rng(d)
    a = rng.standard_normal((1024, d)) * np.linspace(0.2, 3.0, d)
    h = 2 * a.T @ a + np.diag(rng.uniform(0.5, 2.0, d))
    R, info, lam = G.prepare_hchol(torch.from_numpy(h).to(DEV), 0.01, r_dtype=torch.float64)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    hd_o, lam_o = O.damp(h, 0.01)
    ro = O.hessian_factor(hd_o)
    rg = R.cpu().numpy()
    rel = np.linalg.norm(rg - ro) / np.linalg.norm(ro)
    say(f"  R rel={rel:.3e}")
    assert np.all(np.tril(rg, -1) == 0)
    assert rel <= 1e-12
    assert abs(float(lam.item()) - lam_o) <= 1e-12 * lam_o


@pytest.mark.parametrize("d,r_dtype", [(768, torch.float64), (768, torch.float32), (40, torch.float64),
                                       (1000, torch.float64), (8256, torch.float64), (1537, torch.float64)])
def test_hchol_parity(d, r_dtype):
    """gptq_prepare_hchol: R (R R^T = H_d) against the oracle's hessian_factor."""
    say(f"[case] hchol d={d} r_dtype={r_dtype}")
    rng = np.random.default_rng(d + 7)
    a = rng.standard_normal((4 * d, d)) @ np.diag(1.0 / np.arange(1, d + 1)) @ np.linalg.qr(rng.standard_normal((d, d)))[0]
    h = 2 * a.T @ a
    R, info, lam = G.prepare_hchol(torch.from_numpy(h).to(DEV), 0.01, r_dtype=r_dtype)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    hd_o, lam_o = O.damp(h, 0.01)
    ro = O.hessian_factor(hd_o)
    rg = R.cpu().double().numpy()
    rel = np.linalg.norm(rg - ro) / np.linalg.norm(ro)
    say(f"  R rel={rel:.3e}")
    assert np.all(np.tril(rg, -1) == 0)
    assert rel <= (1e-12 if r_dtype == torch.float64 else 2e-7)
    assert abs(float(lam.item()) - lam_o) <= 1e-12 * lam_o
    # diagonal H_d: R = diag(sqrt(h)); H = 0 without damping is not positive definite
    dg = np.linspace(1.0, 9.0, 128)
    R2, info2, _ = G.prepare_hchol(torch.from_numpy(np.diag(dg)).to(DEV), 0.0)
    Z, info3, _ = G.prepare_hchol(torch.zeros(128, 128, dtype=torch.float64, device=DEV), 0.0)
    torch.cuda.synchronize()
    assert int(info2.item()) == 0 and int(info3.item()) > 0
    np.testing.assert_allclose(R2.cpu().numpy(), np.diag(np.sqrt(dg)), rtol=1e-15, atol=0)


def test_chain_diagonal_and_not_positive_definite():
    say("[case] chain diagonal / non-PD")
    d = 128
    diag = np.linspace(1.0, 9.0, d)
    U, info, _ = G.prepare_hinv(torch.from_numpy(np.diag(diag)).to(DEV), 0.0, u_dtype=torch.float64)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    np.testing.assert_allclose(U.cpu().numpy(), np.diag(diag ** -0.5), rtol=1e-14, atol=0)
    # all-zero H without damping is not positive definite
    U, info, _ = G.prepare_hinv(torch.zeros(d, d, dtype=torch.float64, device=DEV), 0.0)
    torch.cuda.synchronize()
    assert int(info.item()) > 0
    with pytest.raises(np.linalg.LinAlgError):
        O.inverse_hessian_factor(np.zeros((d, d)))


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------
def _layer_case(cfg, chunk_tokens=None, label=None, factor="U"):
    say(f"[case] layer {label or cfg.name} m={cfg.m} d={cfg.d} n={cfg.n_tokens} bits={cfg.bits} "
        f"grid={cfg.grid} group={cfg.group} factor={factor}")
    w, x = S.make_layer(cfg, device=S.default_device_for(cfg))
    w, x = w.cpu(), x.cpu()
    gpu = gpu_layer(w, x, cfg.bits, cfg.group, cfg.grid, cfg.damp, chunk_tokens=chunk_tokens, factor=factor)
    stats = compare_layer(w, x, cfg.bits, cfg.group, cfg.grid, gpu, cfg.damp, (label or cfg.name) + f" [{factor}]")
    assert_gates(stats)
    return stats


@pytest.mark.parametrize("factor", ["U", "R"])
def test_layer_parity_toy768(factor):
    _layer_case(S.CONFIGS["toy768"], factor=factor)


_SCALED = [
    ("attn-3b-g128", S.scaled(S.CONFIGS["opt13b-attn"], m=512, d=1024, n_tokens=16384)),
    ("fc1-2b-g128", S.scaled(S.CONFIGS["opt175b-fc1-2bit"], m=512, d=1024, n_tokens=16384)),
    ("fc1-ternary-g128", S.scaled(S.CONFIGS["opt175b-fc1-ternary"], m=512, d=1024, n_tokens=16384)),
    ("4b-g32-ragged-m", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=1000, d=512, n_tokens=8192, group=32)),
    ("4b-g64", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=256, d=512, n_tokens=8192, group=64)),
    ("3b-g256-multiblock", S.scaled(S.CONFIGS["opt13b-attn"], m=256, d=1024, n_tokens=8192, group=256)),
    ("3b-row-d96-ragged-n", S.scaled(S.CONFIGS["opt13b-attn"], m=200, d=96, n_tokens=3000, group=0)),
    ("2b-g32-d224", S.scaled(S.CONFIGS["opt175b-fc1-2bit"], m=130, d=224, n_tokens=5000, group=32)),
    ("8b-row", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=128, d=256, n_tokens=4096, bits=8)),
    ("3b-sym-g128", S.scaled(S.CONFIGS["opt13b-attn"], m=256, d=1024, n_tokens=8192, grid="sym")),
    ("4b-sym-row", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=300, d=512, n_tokens=8192, grid="sym")),
    ("4b-sym-g32", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=200, d=512, n_tokens=8192, grid="sym", group=32)),
    # several super-blocks with a ragged last block, and groups of three blocks
    ("3b-g32-d992-ragged", S.scaled(S.CONFIGS["opt13b-attn"], m=300, d=992, n_tokens=8192, group=32)),
    ("4b-g384-d1152", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=192, d=1152, n_tokens=8192, group=384)),
    # groups not aligned to the 128-column block: 16 inside a lane's columns; 96 and 192 cut the lazy blocks
    ("3b-g16", S.scaled(S.CONFIGS["opt13b-attn"], m=256, d=512, n_tokens=8192, group=16)),
    ("4b-g96-d480", S.scaled(S.CONFIGS["opt2.7b-fc1"], m=200, d=480, n_tokens=8192, group=96)),
    ("3b-g192-d768", S.scaled(S.CONFIGS["opt13b-attn"], m=160, d=768, n_tokens=8192, group=192)),
    ("2b-g160-d1280", S.scaled(S.CONFIGS["opt175b-fc1-2bit"], m=128, d=1280, n_tokens=8192, group=160)),
]


@pytest.mark.parametrize("label,cfg", _SCALED, ids=[c[0] for c in _SCALED])
def test_layer_parity_scaled(label, cfg):
    _layer_case(cfg, label=label)


# the R form (factor R = U^-1): every group size it takes (groups above 128 need U)
_SCALED_R = [(label, cfg) for label, cfg in _SCALED if cfg.group in (0, 16, 32, 64, 128)]


@pytest.mark.parametrize("label,cfg", _SCALED_R, ids=[c[0] for c in _SCALED_R])
def test_layer_parity_scaled_rform(label, cfg):
    _layer_case(cfg, label=label, factor="R")


def test_rform_rejects_groups_wider_than_a_block():
    lib = G.load_library()
    import ctypes
    cfg = G.make_qcfg(4, group_size=256, factor="R")
    w = torch.zeros(8, 512, dtype=torch.float16, device=DEV)
    R = torch.eye(512, dtype=torch.float64, device=DEV)
    out = torch.empty(8, 64, dtype=torch.int32, device=DEV)
    sc = torch.empty(8, 2, dtype=torch.float32, device=DEV)
    zz = torch.empty(8, 2, dtype=torch.uint8, device=DEV)
    st = lib.gptq_quantize_layer(G._ptr(w), G.GPTQ_F16, 8, 512, 512, G._ptr(R), G.GPTQ_F64, 512, ctypes.byref(cfg),
                                 G._ptr(out), G._ptr(sc), G._ptr(zz), None, None, G._ptr(w), 1 << 20, G._stream(DEV))
    assert st == G.GPTQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("factor", ["U", "R"])
def test_layer_parity_d12288_slice(factor):
    """OPT-175B q/k/v/out width (d = 12288) on 64 rows and 16384 tokens: the
    conditioning of the full layer, at a size the oracle finishes quickly."""
    cfg = S.scaled(S.CONFIGS["opt175b-q"], m=64, n_tokens=16384)
    _layer_case(cfg, chunk_tokens=8192, label="opt175b-q-slice", factor=factor)


def test_rtn_reduction_on_gpu():
    """Hadamard tokens make H = 2N I: U is exactly diagonal, nothing propagates,
    and the GPU codes are round-to-nearest codes."""
    say("[case] RTN reduction (Hadamard X)")
    n, d, m = 256, 128, 64
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    x = torch.from_numpy(h[:, :d].astype(np.float16))
    w = torch.from_numpy((np.random.default_rng(3).standard_normal((m, d)) * 0.02).astype(np.float32))
    for group in (0, 32):
        gpu = gpu_layer(w, x, 4, group, "asym")
        assert np.all(np.triu(gpu["U"], 1) == 0)
        rtn = O.rtn_quantize(w.double().numpy(), 4, "asym", group)
        differ = gpu["codes"] != rtn.codes
        assert np.all(rtn.dist[differ] < 1e-5), np.sum(differ)


def test_determinism_bitwise():
    cfg = S.scaled(S.CONFIGS["opt13b-attn"], m=256, d=512, n_tokens=8192)
    say("[case] determinism two runs")
    w, x = S.make_layer(cfg, device="cuda")
    w, x = w.cpu(), x.cpu()
    a = gpu_layer(w, x, cfg.bits, cfg.group, cfg.grid)
    b = gpu_layer(w, x, cfg.bits, cfg.group, cfg.grid)
    for k in ("H", "U", "qcodes", "scales", "zeros", "w_hat", "err_sq"):
        assert np.array_equal(a[k], b[k]), k


def test_workspace_too_small_is_reported():
    say("[case] workspace too small")
    w = torch.zeros(64, 128, dtype=torch.float16, device=DEV)
    U = torch.eye(128, dtype=torch.float32, device=DEV)
    with pytest.raises(G.GPTQError, match="WORKSPACE"):
        _call_with_small_ws(w, U)


def _call_with_small_ws(w, U):
    lib = G.load_library()
    import ctypes
    cfg = G.make_qcfg(4)
    out = torch.empty(64, 16, dtype=torch.int32, device=DEV)
    sc = torch.empty(64, 1, dtype=torch.float32, device=DEV)
    zz = torch.empty(64, 1, dtype=torch.uint8, device=DEV)
    ws = torch.empty(4096, dtype=torch.uint8, device=DEV)
    st = lib.gptq_quantize_layer(G._ptr(w), G.GPTQ_F16, 64, 128, 128, G._ptr(U), G.GPTQ_F32, 128, ctypes.byref(cfg),
                                 G._ptr(out), G._ptr(sc), G._ptr(zz), None, None, G._ptr(ws), 4096,
                                 G._stream(DEV))
    G._check(st, "gptq_quantize_layer")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("factor", ["U", "R"])
def test_layer_parity_opt27b_fc1_full(factor):
    """OPT-2.7B fc1 at full size (10240 x 2560, 262144 tokens, 4-bit per row),
    in the launch configuration the benchmark times (one call over all 262144
    tokens)."""
    _layer_case(S.CONFIGS["opt2.7b-fc1"], chunk_tokens=262144, factor=factor)


def test_prepare_hinv_u_may_alias_h():
    """U written over H's own buffer (the chain copies H into its workspace
    before U is stored) equals U in a separate buffer, bit for bit, for fp64
    and fp32 outputs."""
    say("[case] U aliasing H")
    cfg = S.scaled(S.CONFIGS["opt13b-attn"], m=64, d=416, n_tokens=4096)
    x = S.make_activations(cfg).to(DEV)
    d = cfg.d
    H = torch.empty(d, d, dtype=torch.float64, device=DEV)
    G.accumulate_hessian(H, x, accumulate=False)
    for u_dtype in (torch.float64, torch.float32):
        U_sep, info, lam = G.prepare_hinv(H, 0.01, u_dtype=u_dtype)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        Hc = H.clone()
        if u_dtype == torch.float64:
            U_al = Hc
        else:
            U_al = Hc.view(torch.float32)[:, :d]  # fp32 rows over the fp64 rows, ld = 2 d
        _, info2, lam2 = G.prepare_hinv(Hc, 0.01, U=U_al)
        torch.cuda.synchronize()
        assert int(info2.item()) == 0 and float(lam2.item()) == float(lam.item())
        assert torch.equal(U_al, U_sep), u_dtype
