"""Sequential quantization of one OPT decoder block: every linear layer is
calibrated on the inputs that the block's already quantized layers produce.

FDE Interviews breakdown of GPTQ, figure "Quantize a column, correct the rest"
(caption): the model is quantized one Transformer block at a time on the GPU;
within the block, the layers are quantized in the order the forward pass
reaches them, and the inputs of a layer are computed with the quantized
weights of the layers before it.

This is harness code around the library: the block's forward pass between the
quantizations (LayerNorm, the projections with the dequantized weights,
causal attention per sequence, ReLU) runs in plain torch on the GPU; every
step of the quantization itself runs in the library's kernels (gptq.py).

The block is OPT's decoder layer (pre-LayerNorm):
    a = LN1(x);  q, k, v = a Wq^T, a Wk^T, a Wv^T
    o = causal multi-head attention(q, k, v) within each sequence
    h = x + o Wo^T
    f = LN2(h);  u = ReLU(f W1^T);  y = h + u W2^T
with synthetic weights (the generator's W for each sublayer, no biases,
LayerNorm gain 1 and shift 0). Layers and their calibration inputs:
    q, k, v   LN1(x)                          (one Hessian, one factor)
    out       attention output, from the quantized q, k, v
    fc1       LN2(h), h from the quantized out
    fc2       ReLU(LN2(h) W1_hat^T), from the quantized fc1
Products take fp16 operands with fp32 accumulation; LayerNorm, the attention
scores and the softmax are fp32; activations are stored in fp16, the dtype
the Hessian accumulation takes.
"""

from __future__ import annotations

import dataclasses
import math

import torch

from . import gptq as G
from . import synthetic as S


@dataclasses.dataclass(frozen=True)
class BlockShape:
    d_model: int
    n_heads: int
    d_ffn: int
    seq_len: int
    n_tokens: int
    bits: int = 3
    group: int = 128
    grid: str = "asym"
    damp: float = 0.01


# OPT-175B: hidden 12288, 96 heads of 128, ffn 49152; 128 sequences of 2048 tokens
OPT175B = BlockShape(12288, 96, 49152, S.SEQ_LEN, 128 * S.SEQ_LEN)

SUBLAYERS = ["q", "k", "v", "out", "fc1", "fc2"]


def layer_configs(shape: BlockShape):
    """The generator's configurations of the six sublayers at this shape (W
    seeds from the OPT-175B block's configurations, resized)."""
    base = {"q": "opt175b-q", "k": "opt175b-k", "v": "opt175b-v", "out": "opt175b-out",
            "fc1": "opt175b-fc1", "fc2": "opt175b-fc2"}
    dims = {"q": (shape.d_model, shape.d_model), "k": (shape.d_model, shape.d_model),
            "v": (shape.d_model, shape.d_model), "out": (shape.d_model, shape.d_model),
            "fc1": (shape.d_ffn, shape.d_model), "fc2": (shape.d_model, shape.d_ffn)}
    out = {}
    for name in SUBLAYERS:
        m, d = dims[name]
        c = S.CONFIGS[base[name]]
        out[name] = c if (c.m, c.d, c.n_tokens) == (m, d, shape.n_tokens) and (c.bits, c.group, c.grid) == (
            shape.bits, shape.group, shape.grid) else S.scaled(c, m=m, d=d, n_tokens=shape.n_tokens,
                                                                 bits=shape.bits, group=shape.group, grid=shape.grid)
    return out


def block_input(shape: BlockShape, device) -> torch.Tensor:
    """The block's input hidden states x [n_tokens, d_model] fp16: the
    generator's correlated activations of the q layer's configuration."""
    return S.make_activations(layer_configs(shape)["q"], device)


def layer_norm(x: torch.Tensor, chunk: int = 16384) -> torch.Tensor:
    """LayerNorm over the hidden dimension (gain 1, shift 0, eps 1e-5) in fp32,
    returned in fp16."""
    out = torch.empty_like(x, dtype=torch.float16)
    for t0 in range(0, x.shape[0], chunk):
        xs = x[t0:t0 + chunk].float()
        mu = xs.mean(dim=1, keepdim=True)
        var = ((xs - mu) ** 2).mean(dim=1, keepdim=True)
        out[t0:t0 + chunk] = ((xs - mu) * torch.rsqrt(var + 1e-5)).half()
    return out


def linear(x: torch.Tensor, w_hat: torch.Tensor, chunk: int = 32768) -> torch.Tensor:
    """x W_hat^T with fp16 operands and fp32 accumulation, fp16 result [n, m]."""
    wt = w_hat.t().contiguous().half()
    out = torch.empty(x.shape[0], w_hat.shape[0], dtype=torch.float16, device=x.device)
    for t0 in range(0, x.shape[0], chunk):
        out[t0:t0 + chunk] = torch.matmul(x[t0:t0 + chunk], wt)
    return out


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_heads: int, seq_len: int,
              seqs_per_chunk: int = 2) -> torch.Tensor:
    """Causal multi-head attention within each sequence of seq_len tokens
    (q, k, v [n_tokens, d] fp16; scores and softmax in fp32), fp16 output."""
    n, d = q.shape
    dh = d // n_heads
    out = torch.empty_like(q)
    mask = torch.triu(torch.ones(seq_len, seq_len, dtype=torch.bool, device=q.device), diagonal=1)
    scale = 1.0 / math.sqrt(dh)
    step = seqs_per_chunk * seq_len
    for t0 in range(0, n, step):
        t1 = min(t0 + step, n)
        ns = (t1 - t0) // seq_len

        def heads(t):
            return t[t0:t1].float().view(ns, seq_len, n_heads, dh).permute(0, 2, 1, 3).contiguous()
        qh, kh, vh = heads(q), heads(k), heads(v)
        kt = kh.transpose(-1, -2).contiguous()
        sc = torch.matmul(qh, kt) * scale
        sc.masked_fill_(mask, float("-inf"))
        p = torch.softmax(sc, dim=-1)
        o = torch.matmul(p, vh)                                   # [ns, H, seq, dh]
        out[t0:t1] = o.permute(0, 2, 1, 3).reshape(t1 - t0, d).half()
    return out


class SequentialBlock:
    """Quantizes the six sublayers of one block in forward order through the
    library (H, the R factor, the column loop), computing each sublayer's
    calibration input from the sublayers quantized before it. `inputs` keeps
    the calibration input of every sublayer (q, k and v share one)."""

    def __init__(self, shape: BlockShape, device, factor: str = "R"):
        self.shape = shape
        self.device = torch.device(device)
        self.factor = factor
        self.cfgs = layer_configs(shape)
        self.weights = {n: S.make_weights(c, self.device) for n, c in self.cfgs.items()}
        self.results = {}
        self.inputs = {}
        self.stage_s = {}

    def _quantize(self, names, x):
        d = x.shape[1]
        H = torch.empty(d, d, dtype=torch.float64, device=self.device)
        G.accumulate_hessian(H, x, accumulate=False)
        c0 = self.cfgs[names[0]]
        if self.factor == "R":
            F, info, lam = G.prepare_hchol(H, c0.damp)
        else:
            F, info, lam = G.prepare_hinv(H, c0.damp)
        if int(info.item()) != 0:
            raise RuntimeError(f"H + lambda I of {names} is not positive definite")
        for n in names:
            c = self.cfgs[n]
            self.results[n] = G.quantize_layer(self.weights[n], F, c.bits, c.group, c.grid, factor=self.factor)
        del H, F

    def run(self, x: torch.Tensor):
        """x: the block input [n_tokens, d_model] fp16. Returns the block output
        y computed with every sublayer quantized."""
        sh = self.shape
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(9)]
        ev[0].record()
        a = layer_norm(x)
        self.inputs["q"] = self.inputs["k"] = self.inputs["v"] = a
        ev[1].record()
        self._quantize(["q", "k", "v"], a)
        ev[2].record()
        q, k, v = (linear(a, self.results[n]["w_hat"]) for n in ("q", "k", "v"))
        o = attention(q, k, v, sh.n_heads, sh.seq_len)
        del q, k, v
        self.inputs["out"] = o
        ev[3].record()
        self._quantize(["out"], o)
        ev[4].record()
        h = (x.float() + linear(o, self.results["out"]["w_hat"]).float()).half()
        f = layer_norm(h)
        self.inputs["fc1"] = f
        ev[5].record()
        self._quantize(["fc1"], f)
        ev[6].record()
        u = torch.relu(linear(f, self.results["fc1"]["w_hat"]))
        self.inputs["fc2"] = u
        ev[7].record()
        self._quantize(["fc2"], u)
        ev[8].record()
        y = (h.float() + linear(u, self.results["fc2"]["w_hat"]).float()).half()
        torch.cuda.synchronize()
        el = [ev[i].elapsed_time(ev[i + 1]) for i in range(8)]
        self.stage_s = {"forward_ms": el[0] + el[2] + el[4] + el[6],
                        "quantize_ms": {"qkv": el[1], "out": el[3], "fc1": el[5], "fc2": el[7]}}
        return y
