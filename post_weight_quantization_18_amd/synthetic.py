"""Seeded synthetic layers: weights W and calibration activations X.

This module only draws inputs. It holds none of the quantization method's
arithmetic, and it serves both the GPU path (tests, bench) and the CPU oracle,
which receive the same tensors.

The real workloads are OPT/BLOOM layers calibrated on 128 sequences x 2048
tokens of web text (FDE Interviews breakdown of GPTQ, figure "Quantize a column,
correct the rest": "128 C4 sequences of 2,048 tokens"). No weights or datasets
are used here; the inputs take the workloads' shapes and the structure the
method relies on, correlated input channels (section 01: another weight can
absorb the damage because inputs are correlated), plus a few outlier channels.

Recipe (all seeds derive from (config, layer, stream, chunk)):

* W [m, d]: iid N(0, 0.02^2); 8 distinct input columns scaled x10; cast
  round-to-nearest-even to fp32 or fp16.
* X [N, d] fp16 = Z A per 2048-token sequence, Z iid N(0, 1),
  A = diag(s) Q^T with Q Haar-orthogonal (QR of a Gaussian, sign-fixed),
  s_k = c / k (k = 1..d) with c chosen so the mean channel variance is 1, and
  6 distinct channels (columns of A) scaled x20.
  For d > 16384 (the OPT-175B fc2 input width) a dense Haar Q costs more than
  the rest of the run, so Q = P2 B2 P1 B1 instead: B1, B2 block-diagonal with
  Haar blocks of 4096, P1, P2 random permutations. The spectrum s is the same,
  so the conditioning of H is too; only the mixing pattern is structured.

The orthogonal factors (Q, or the Haar blocks of the structured Q) are
always drawn on the CPU in fp64 (torch's CPU generator and LAPACK QR), whatever
the device, so they do not depend on the GPU or its solver libraries. Small
configurations then form X on the CPU in fp64; large ones form it on the GPU
(Q cast to fp32, fp32 GEMM per sequence), which is fast and deterministic for a
given device type. Either way the same fp16 X goes to both sides of a parity
test.

The two grids of the extreme regime (2-bit and ternary on the OPT-175B fc1
shape) quantize one layer: they share W and X (the same seeds).
"""

from __future__ import annotations

import dataclasses
import math

import torch

SEQ_LEN = 2048


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    m: int            # output features (rows of W)
    d: int            # input features (columns of W)
    n_tokens: int     # calibration tokens
    w_dtype: str      # "fp32" | "fp16"
    bits: int
    grid: str         # "asym" | "ternary" | "sym"
    group: int        # 0 = per output row
    block: int = 128
    damp: float = 0.01
    config_id: int = 0
    layer_id: int = 0

    @property
    def n_weights(self) -> int:
        return self.m * self.d


def _cfg(name, m, d, n, wdt, bits, grid, group, cid, lid=0):
    return LayerConfig(name, m, d, n, wdt, bits, grid, group, config_id=cid, layer_id=lid)


_N = 128 * SEQ_LEN  # 262144 calibration tokens

CONFIGS = {
    # toy layer, 2 sequences
    "toy768": _cfg("toy768", 768, 768, 2 * SEQ_LEN, "fp32", 4, "asym", 0, 1),
    # OPT-2.7B fc1
    "opt2.7b-fc1": _cfg("opt2.7b-fc1", 10240, 2560, _N, "fp16", 4, "asym", 0, 2),
    # OPT-13B attention projection
    "opt13b-attn": _cfg("opt13b-attn", 5120, 5120, _N, "fp16", 3, "asym", 128, 3),
    # OPT-175B block: six layers, each its own X
    "opt175b-q": _cfg("opt175b-q", 12288, 12288, _N, "fp16", 3, "asym", 128, 4, 0),
    "opt175b-k": _cfg("opt175b-k", 12288, 12288, _N, "fp16", 3, "asym", 128, 4, 1),
    "opt175b-v": _cfg("opt175b-v", 12288, 12288, _N, "fp16", 3, "asym", 128, 4, 2),
    "opt175b-out": _cfg("opt175b-out", 12288, 12288, _N, "fp16", 3, "asym", 128, 4, 3),
    "opt175b-fc1": _cfg("opt175b-fc1", 49152, 12288, _N, "fp16", 3, "asym", 128, 4, 4),
    "opt175b-fc2": _cfg("opt175b-fc2", 12288, 49152, _N, "fp16", 3, "asym", 128, 4, 5),
    # extreme regime on the OPT-175B fc1 shape
    "opt175b-fc1-2bit": _cfg("opt175b-fc1-2bit", 49152, 12288, _N, "fp16", 2, "asym", 128, 5, 0),
    "opt175b-fc1-ternary": _cfg("opt175b-fc1-ternary", 49152, 12288, _N, "fp16", 2, "ternary", 128, 5, 0),
}

OPT175B_BLOCK = ["opt175b-q", "opt175b-k", "opt175b-v", "opt175b-out", "opt175b-fc1", "opt175b-fc2"]


def scaled(cfg: LayerConfig, m=None, d=None, n_tokens=None, **kw) -> LayerConfig:
    """The same recipe at other sizes (parity cases that the oracle finishes fast)."""
    return dataclasses.replace(cfg, name=cfg.name + "-scaled", m=m or cfg.m, d=d or cfg.d,
                               n_tokens=n_tokens or cfg.n_tokens, **kw)


def _seed(cfg: LayerConfig, stream: int, chunk: int = 0) -> int:
    v = (((cfg.config_id * 131 + cfg.layer_id) * 1009 + stream) * 1_000_003 + chunk)
    v ^= (cfg.m * 2654435761) & 0xFFFFFFFF
    v ^= (cfg.d * 40503) << 7
    return v & 0x7FFF_FFFF_FFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_weights(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    """W [m, d] in cfg.w_dtype."""
    dev = torch.device(device)
    work = torch.float64 if dev.type == "cpu" else torch.float32
    w = torch.randn(cfg.m, cfg.d, generator=_gen(dev, _seed(cfg, 0)), device=dev, dtype=work) * 0.02
    gi = _gen(torch.device("cpu"), _seed(cfg, 1))
    n_out = min(8, cfg.d)
    cols = torch.randperm(cfg.d, generator=gi)[:n_out].to(dev)
    w[:, cols] *= 10.0
    return w.to(torch.float32 if cfg.w_dtype == "fp32" else torch.float16)


STRUCTURED_D = 16384
BLOCK_Q = 4096


def _haar(n, gen, dev, work):
    """Haar-distributed orthogonal n x n matrix: QR of an fp64 Gaussian drawn
    with the CPU generator `gen`, columns sign-fixed by diag(R); computed on
    the CPU, then moved to `dev` in `work` precision."""
    g = torch.randn(n, n, generator=gen, dtype=torch.float64)
    q, r = torch.linalg.qr(g)
    q = q * torch.sign(torch.diagonal(r)).unsqueeze(0)
    return q.to(device=dev, dtype=work)


def _spectrum(d, dev, work):
    k = torch.arange(1, d + 1, device=dev, dtype=work)
    c = math.sqrt(d / float(torch.sum(1.0 / (k.double().cpu() ** 2))))
    return c / k


def _outlier_channels(cfg, dev):
    gi = _gen(torch.device("cpu"), _seed(cfg, 3))
    return torch.randperm(cfg.d, generator=gi)[:min(6, cfg.d)].to(dev)


def mixing_matrix(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    """A = diag(s) Q^T with 6 outlier channels x20 (fp64 on CPU, fp32 on GPU);
    dense Haar Q (d <= 16384 only)."""
    dev = torch.device(device)
    work = torch.float64 if dev.type == "cpu" else torch.float32
    d = cfg.d
    assert d <= STRUCTURED_D, "the dense mixing matrix is only drawn up to d = 16384"
    q = _haar(d, _gen(torch.device("cpu"), _seed(cfg, 2)), dev, work)
    a = _spectrum(d, dev, work).unsqueeze(1) * q.t()
    a[:, _outlier_channels(cfg, dev)] *= 20.0
    return a.contiguous()


class _StructuredMix:
    """x -> x diag(s) Q^T with Q = P2 B2 P1 B1 (see the module docstring), then
    the outlier channels x20; applied to row blocks of Z."""

    def __init__(self, cfg, dev, work):
        d = cfg.d
        assert d % BLOCK_Q == 0
        nb = d // BLOCK_Q
        gq = _gen(torch.device("cpu"), _seed(cfg, 2))
        self.b1 = torch.stack([_haar(BLOCK_Q, gq, dev, work) for _ in range(nb)])
        self.b2 = torch.stack([_haar(BLOCK_Q, gq, dev, work) for _ in range(nb)])
        gp = _gen(torch.device("cpu"), _seed(cfg, 5))
        self.p1 = torch.randperm(d, generator=gp).to(dev)
        self.p2 = torch.randperm(d, generator=gp).to(dev)
        self.s = _spectrum(d, dev, work)
        self.chans = _outlier_channels(cfg, dev)
        self.nb = nb

    def _blockmul_t(self, y, b):
        # y [t, d] times blockdiag(b)^T
        t = y.shape[0]
        yb = y.view(t, self.nb, BLOCK_Q).transpose(0, 1)           # [nb, t, 4096]
        out = torch.bmm(yb, b.transpose(1, 2).contiguous())         # [nb, t, 4096]
        return out.transpose(0, 1).reshape(t, -1)

    def __call__(self, z):
        # Q^T = B1^T P1^T B2^T P2^T; a permutation P (x P = x[:, perm]) acts
        # on the right as a column gather
        y = z * self.s
        y = self._blockmul_t(y, self.b1)
        y = y[:, torch.argsort(self.p1)]
        y = self._blockmul_t(y, self.b2)
        y = y[:, torch.argsort(self.p2)]
        y[:, self.chans] *= 20.0
        return y


def make_activations(cfg: LayerConfig, device="cpu", out=None) -> torch.Tensor:
    """X [N, d] fp16, token-major, drawn sequence by sequence."""
    dev = torch.device(device)
    work = torch.float64 if dev.type == "cpu" else torch.float32
    if cfg.d > STRUCTURED_D:
        mix = _StructuredMix(cfg, dev, work)
    else:
        a = mixing_matrix(cfg, dev)
        mix = lambda z: z @ a  # noqa: E731
    n = cfg.n_tokens
    if out is None:
        out = torch.empty(n, cfg.d, dtype=torch.float16, device=dev)
    seq = min(SEQ_LEN, n)
    for t0 in range(0, n, seq):
        t1 = min(t0 + seq, n)
        z = torch.randn(t1 - t0, cfg.d, generator=_gen(dev, _seed(cfg, 4, t0 // seq)),
                        device=dev, dtype=work)
        out[t0:t1] = mix(z).to(torch.float16)
    return out


def make_layer(cfg: LayerConfig, device="cpu"):
    """(W, X) on `device`."""
    return make_weights(cfg, device), make_activations(cfg, device)


def default_device_for(cfg: LayerConfig) -> str:
    """CPU for layers the oracle handles quickly, GPU for the large shapes."""
    return "cpu" if cfg.n_tokens * cfg.d <= 4096 * 1024 else "cuda"
