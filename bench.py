"""Benchmark of the GPTQ layer-quantization hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config opt175b-fc2]
                    [--factor auto|R|U] [--act-order [--static-groups]]
    python bench.py --gemv [--act-order] [--steps K] [--warmup W]
    python bench.py --block [--sequential] [--steps K] [--warmup W]
    python bench.py --vendor-gemm | --copy-calibration

One step = the whole hot path on one layer with W and X already resident in
HBM: H accumulated over all of the layer's calibration tokens in one call
(--chunk-tokens splits it into calls of that many tokens, as a caller that
streams its calibration batches would), the fp64 factor (R, the Cholesky
factor of H + lambda I, from d = 8192 on; U = chol(H_d^-1) below, or as
--factor says), then the column loop with lazy 128-column updates, trailing
GEMMs and packing.
With --act-order the step also orders the columns by descending H_jj, gathers
H into that order before the chain, and runs the column loop in that order
(--static-groups: grids fitted on the original weights' natural groups).
--gemv times generation with the packed weights instead: one token through the
six layers of an OPT-175B block (q, k, v, out, fc1, fc2; 3-bit, g128), each a
dequantizing matrix-vector product that streams its packed codes from HBM.
--block times the quantization of a whole OPT-175B block, layer by layer: q, k
and v see the same input, so one Hessian and one factor serve all three; out,
fc1 and fc2 each have their own (synthetic) input.
Prints one JSON line (rank 0). The per-stage device times come from HIP events
recorded on the stream the library launches on (torch's current stream). The
timed steps also run under the library's trace (gptq_trace_start / stop), which
brackets every kernel launch with HIP events on its launch stream, so that the
line reports the device time, launch count and roofline fraction of each kernel
family (SYRK, trailing GEMM, fp64 chain, column loop) over the timed region.
The default workload is the OPT-175B fc2 layer (12288 x 49152, 262144
calibration tokens, 3-bit asymmetric g128).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

from post_weight_quantization_18_amd import gptq as G
from post_weight_quantization_18_amd import synthetic as S

PEAK_FP16_TFLOPS = 2516.6     # MI355X dense fp16/bf16 MFMA, fp32 accumulate
PEAK_FP64_TFLOPS = 78.6       # MI355X fp64 (vector and matrix)
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP32_VECTOR_TFLOPS = 157.3   # MI355X fp32 vector
CHUNK_TOKENS = 262144         # the whole calibration set (128 sequences of 2048) per accumulate call

# HBM traffic of one SYRK launch (syrk_kernel<true>, the feature-major form) at
# the default workload, from two
# rocprofv3 --pmc passes over this command (FETCH_SIZE, WRITE_SIZE, KiB per
# dispatch), each scaled by what the counter reads for a 1 GiB copy (FETCH_SIZE
# x2.0, WRITE_SIZE x1.0); see profiles/syrk_kernel_opt175b-fc2_traffic.md. The
# figure is only reported while the kernel source is the one it was taken on.
SYRK_TRAFFIC = {
    "config": "opt175b-fc2",
    "chunk_tokens": 262144,
    "source_sha256_16": "52974eca4cb9822b",   # syrk.hip + common.h
    "fetch_bytes": 176326002.7 * 1024 * 2.0,
    "write_bytes": 9488112.0 * 1024 * 1.0,
}


def _syrk_source_hash():
    import hashlib
    h = hashlib.sha256()
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "post_weight_quantization_18_amd", "csrc")
    for f in ("syrk.hip", "common.h"):
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def syrk_traffic(cfg_name, chunk):
    t = SYRK_TRAFFIC
    if cfg_name != t["config"] or chunk != t["chunk_tokens"] or _syrk_source_hash() != t["source_sha256_16"]:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--config", default="opt175b-fc2", choices=sorted(S.CONFIGS))
    p.add_argument("--factor", choices=["auto", "R", "U"], default="auto",
                   help="auto: R from d = 8192 on (measured faster there: no triangular inverse), U below (the "
                        "R form's fixed costs dominate small layers); "
                        "R: the Cholesky factor of H_d (gptq_prepare_hchol, no inverse); "
                        "U: chol(H_d^-1) (gptq_prepare_hinv)")
    p.add_argument("--no-trace", action="store_true",
                   help="time the steps without the per-kernel trace (no per-family breakdown)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--act-order", action="store_true",
                   help="quantize the columns in descending H_jj (desc_act)")
    p.add_argument("--block", action="store_true",
                   help="time the quantization of a whole OPT-175B block (q, k, v sharing one Hessian)")
    p.add_argument("--sequential", action="store_true",
                   help="with --block: calibrate each sublayer on the block's forward pass through the sublayers "
                        "quantized before it (the block input is synthetic; the forward runs in torch)")
    p.add_argument("--gemv", action="store_true",
                   help="time the dequantizing matrix-vector product over an OPT-175B block instead")
    p.add_argument("--static-groups", action="store_true",
                   help="with --act-order: grids of the natural groups, fitted on the original weights")
    p.add_argument("--chunk-tokens", type=int, default=CHUNK_TOKENS,
                   help="tokens per gptq_accumulate_hessian call (the whole X stays resident either way)")
    p.add_argument("--cpu-sample-rows", type=int, default=None)
    p.add_argument("--cpu-sample-tokens", type=int, default=None)
    p.add_argument("--vendor-gemm", action="store_true",
                   help="time hipBLASLt fp16 GEMMs at large shapes (context for the SYRK's matrix-core fraction)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only copy 1 GiB device-to-device three times (reference for the HBM byte counters)")
    return p.parse_args()


def vendor_gemm():
    """Context for the SYRK's fraction: hipBLASLt fp16 GEMMs (torch.matmul, fp16 in
    and out) at large shapes, HIP events around ten products after three warm-ups."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for m, n, k, tn in [(16384, 16384, 32768, False), (12288, 12288, 32768, True), (49152, 8192, 32768, True)]:
        if tn:
            a = torch.randn(k, m, generator=g, device=dev, dtype=torch.float16)
            b = a if n == m else torch.randn(k, n, generator=g, device=dev, dtype=torch.float16)
            f = (lambda a=a, b=b: torch.matmul(a.t(), b))
        else:
            a = torch.randn(m, k, generator=g, device=dev, dtype=torch.float16)
            b = torch.randn(k, n, generator=g, device=dev, dtype=torch.float16)
            f = (lambda a=a, b=b: torch.matmul(a, b))
        for _ in range(3):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        tf = 2 * m * n * k / (ms * 1e-3) / 1e12
        print(json.dumps({"vendor_gemm": f"{m}x{k} @ {k}x{n} {'TN' if tn else 'NN'} fp16", "ms": round(ms, 3),
                          "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_FP16_TFLOPS, 4)}), flush=True)
        del a, b


def copy_calibration():
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": "3 x 1 GiB device-to-device copies"}), flush=True)


class LayerRun:
    """Preallocated buffers for one layer; step() enqueues the whole hot path."""

    def __init__(self, cfg: S.LayerConfig, w: torch.Tensor, x: torch.Tensor, chunk: int = CHUNK_TOKENS,
                 act_order: bool = False, static_groups: bool = False, factor: str = "R"):
        chunk = min(chunk, cfg.n_tokens)
        self.cfg = cfg
        self.factor = factor
        self.act_order, self.static_groups = act_order, static_groups
        self.w, self.x = w, x
        dev = w.device
        d, m = cfg.d, cfg.m
        self.H = torch.empty(d, d, dtype=torch.float64, device=dev)
        # U = chol(H_d^-1) in fp32, or R (R R^T = H_d) in fp64: the quantizer inverts
        # R's diagonal blocks from it
        self.U = torch.empty(d, d, dtype=torch.float64 if factor == "R" else torch.float32, device=dev)
        if act_order:
            self.perm = torch.empty(d, dtype=torch.int32, device=dev)
            self.Hp = torch.empty(d, d, dtype=torch.float64, device=dev)
        self.chunk = chunk
        self.ws_h = torch.empty(max(1, G.workspace_bytes(G.WS_ACCUMULATE_HESSIAN, 0, d, chunk)),
                                dtype=torch.uint8, device=dev)
        self.ws_c = torch.empty(G.workspace_bytes(G.WS_PREPARE_HINV, 0, d), dtype=torch.uint8, device=dev)
        qcfg = G.make_qcfg(cfg.bits, cfg.group, cfg.grid, factor=factor)
        self.ws_q = torch.empty(G.workspace_bytes(G.WS_QUANTIZE_LAYER, m, d, 0, qcfg), dtype=torch.uint8, device=dev)
        ng = d // cfg.group if cfg.group else 1
        self.out = {
            "qcodes": torch.empty(m, d * cfg.bits // 32, dtype=torch.int32, device=dev),
            "scales": torch.empty(m, ng, dtype=torch.float32, device=dev),
            "zeros": torch.empty(m, ng, dtype=torch.uint8, device=dev),
            "w_hat": torch.empty(m, d, dtype=torch.float32, device=dev),
            "err_sq": torch.empty(m, dtype=torch.float32, device=dev),
        }
        if act_order:
            self.out["g_idx"] = torch.empty(d, dtype=torch.int32, device=dev)
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        self.ev_h = [torch.cuda.Event(enable_timing=True) for _ in range(2 * self.n_chunks())]
        self.info = None

    def n_chunks(self):
        return (self.cfg.n_tokens + self.chunk - 1) // self.chunk

    def step(self, timed_chunks=False):
        cfg = self.cfg
        self.ev[0].record()
        for i in range(self.n_chunks()):
            t0 = i * self.chunk
            if timed_chunks:
                self.ev_h[2 * i].record()
            G.accumulate_hessian(self.H, self.x[t0:t0 + self.chunk], accumulate=i > 0, workspace=self.ws_h)
            if timed_chunks:
                self.ev_h[2 * i + 1].record()
        self.ev[1].record()
        h = self.H
        if self.act_order:
            G.act_order(self.H, self.perm)
            h = G.permute_hessian(self.H, self.perm, self.Hp)
        self.ev[4].record()
        if self.factor == "R":
            _, self.info, self.lam = G.prepare_hchol(h, cfg.damp, R=self.U, workspace=self.ws_c)
        else:
            _, self.info, self.lam = G.prepare_hinv(h, cfg.damp, U=self.U, workspace=self.ws_c)
        self.ev[2].record()
        if self.act_order:
            G.quantize_layer_ordered(self.w, self.U, self.perm, cfg.bits, cfg.group, cfg.grid, self.static_groups,
                                     workspace=self.ws_q, out=self.out, factor=self.factor)
        else:
            G.quantize_layer(self.w, self.U, cfg.bits, cfg.group, cfg.grid, workspace=self.ws_q, out=self.out,
                             factor=self.factor)
        self.ev[3].record()

    def stage_ms(self):
        st = {"hessian": self.ev[0].elapsed_time(self.ev[1])}
        if self.act_order:
            st["act_order"] = self.ev[1].elapsed_time(self.ev[4])
        st.update({"hinv_chain": self.ev[4].elapsed_time(self.ev[2]), "quantize": self.ev[2].elapsed_time(self.ev[3]),
                   "total": self.ev[0].elapsed_time(self.ev[3])})
        return st

    def syrk_call_ms(self):
        return [self.ev_h[2 * i].elapsed_time(self.ev_h[2 * i + 1]) for i in range(self.n_chunks())]


def _say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cfg, w, x, rows=None, tokens=None, act_order=False, static_groups=False):
    """The fp64 oracle, as it stands, on a bounded sample of the same layer
    (about 10-30 s of CPU work), extrapolated to the whole layer:
      * H over `tokens` calibration tokens, scaled by N / tokens;
      * the chain (damp, Cholesky, inverse) on the leading d_s x d_s block of
        that H (at most 6144), scaled by (d / d_s)^3;
      * the column loop on `rows` rows at full width, scaled by m / rows. Its
        cost does not depend on U's values, so at d > d_s it runs on a stand-in
        upper-triangular U (unit diagonal, 1e-3 above it).
    With act_order the oracle's order, permuted H and ordered loop are timed
    instead (the order from the sampled H)."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max(i.get("num_threads", 1) for i in info) if info else os.cpu_count()
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    d = cfg.d
    if tokens is None:
        tokens = int(min(16384, max(256, 5e12 / d ** 2)) // 256 * 256)
    if rows is None:
        rows = int(min(512, max(16, 2e11 / d ** 2)))
    rows = min(rows, cfg.m)
    tokens = min(tokens, cfg.n_tokens)
    d_s = min(d, 6144)
    xs = x[:tokens].cpu().numpy()
    ws = w[:rows].double().cpu().numpy()
    t0 = time.perf_counter()
    h = O.hessian([xs[i:i + 4096] for i in range(0, tokens, 4096)])
    t1 = time.perf_counter()
    if act_order:
        perm = O.act_order_perm(h)
        hd, _ = O.damp(h[np.ix_(perm[:d_s], perm[:d_s])], cfg.damp)
    else:
        hd, _ = O.damp(h[:d_s, :d_s], cfg.damp)
    u = O.inverse_hessian_factor(hd)
    t2 = time.perf_counter()
    if d_s < d:
        u = np.triu(np.full((d, d), 1e-3))
        np.fill_diagonal(u, 1.0)
    t3 = time.perf_counter()
    if act_order:
        O.gptq_quantize_ordered(ws, u, perm, cfg.bits, cfg.grid, cfg.group, static_groups)
    else:
        O.gptq_quantize(ws, u, cfg.bits, cfg.grid, cfg.group)
    t4 = time.perf_counter()
    t_h = (t1 - t0) * cfg.n_tokens / tokens
    t_chain = (t2 - t1) * (d / d_s) ** 3
    t_loop = (t4 - t3) * cfg.m / rows
    total = t_h + t_chain + t_loop
    return {
        "value": cfg.n_weights / total,
        "unit": "weights/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{cfg.name}{' act-order' if act_order else ''}: H over {tokens} of {cfg.n_tokens} tokens (x{cfg.n_tokens / tokens:g}); chain on "
                   f"the leading {d_s}x{d_s} block (x{(d / d_s) ** 3:g}); column loop on {rows} of {cfg.m} rows "
                   f"(x{cfg.m / rows:g}); measured {t1 - t0 + t2 - t1 + t4 - t3:.1f} s, extrapolated "
                   f"{total:.1f} s per layer"),
        "stage_s": {"hessian": t_h, "chain": t_chain, "loop": t_loop},
        "cpu": platform.processor() or platform.machine(),
    }


def gemv_bench(args):
    """One step = one token through the six OPT-175B block layers, each
    y = W_hat x from its packed 3-bit g128 codes (synthetic random codes,
    scales and zero points: the time does not depend on their values)."""
    dev = torch.device("cuda:0")
    layers = []
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    for name in S.OPT175B_BLOCK:
        cfg = S.CONFIGS[name]
        m, d, bits, group = cfg.m, cfg.d, cfg.bits, cfg.group
        ng = d // group
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (m, d * bits // 32), dtype=torch.int32, device=dev, generator=gen)
        sc = torch.rand(m, ng, device=dev, generator=gen) * 0.01 + 1e-3
        z = torch.randint(0, 1 << bits, (m, ng), dtype=torch.uint8, device=dev, generator=gen)
        x = torch.randn(d, device=dev, generator=gen).half()
        y = torch.empty(m, dtype=torch.float32, device=dev)
        nbytes = m * d * bits // 8 + m * ng * 5 + d * 2 + m * 4
        perm = None
        if args.act_order:
            # act-order codes: a group index spreading every group over the row,
            # the codes rewritten in group order once (outside the timed steps)
            g_idx = torch.randperm(d, device=dev, generator=gen).to(torch.int32) // group
            q, perm, info = G.gemv_prepare_act_order(q, g_idx.contiguous(), bits, group)
            torch.cuda.synchronize()
            assert int(info.item()) == 0
            perm = (perm, torch.empty(d, dtype=torch.float16, device=dev))
            nbytes += d * 4 + d * 2 * 2     # col_perm, and x gathered into x_perm and read back
        layers.append((name, q, sc, z, bits, group, x, y, nbytes, perm))
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in layers]

    def step(timed):
        for i, (name, q, sc, z, bits, group, x, y, nb, perm) in enumerate(layers):
            if timed:
                ev[i][0].record()
            if perm is None:
                G.dequant_gemv(q, sc, z, bits, group, x, y)
            else:
                G.dequant_gemv_perm(q, sc, z, bits, group, perm[0], x, perm[1], y)
            if timed:
                ev[i][1].record()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    per = {l[0]: 0.0 for l in layers}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        for i, l in enumerate(layers):
            per[l[0]] += ev[i][0].elapsed_time(ev[i][1])
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = {k: v / args.steps for k, v in per.items()}
    total_bytes = sum(l[8] for l in layers)
    big = max(layers, key=lambda l: l[8])
    big_gbs = big[8] / (per[big[0]] * 1e-3) / 1e9
    result = {
        "metric": "tokens per second through one OPT-175B block with 3-bit packed weights (batch 1)",
        "value": 1e3 / ms_step,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u3 codes -> f32 (fp16 x)",
        "data": "synthetic packed codes, scales and zero points of the block's shapes",
        "config": {"workload": "OPT-175B block q, k, v, out (12288x12288), fc1 (49152x12288), fc2 (12288x49152); "
                               "3-bit g128 packed weights, one token"
                               + ("; act-order codes (group index, columns sorted by group, x gathered)"
                                  if args.act_order else ""), "block_bytes": total_bytes},
        "layer_ms": {k: round(v, 5) for k, v in per.items()},
        "block_gbs": round(total_bytes / (sum(per.values()) * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": f"dq_gemv_kernel<3> ({big[0]})", "achieved": round(big_gbs, 1),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(big_gbs / 8000.0, 4), "traffic": None,
                     "per_launch": {"bytes": big[8], "avg_ms": round(per[big[0]], 5)}},
    }
    if not args.no_cpu_baseline:
        _say("timing the oracle on sampled rows of every layer (cpu_baseline)")
        result["cpu_baseline"] = gemv_cpu_baseline(layers)
    print(json.dumps(result), flush=True)


# Sublayers of an OPT-175B block that see the same input: q, k and v read the
# attention input; out, fc1 and fc2 read their own.
BLOCK_GROUPS = [("attn-qkv", ["opt175b-q", "opt175b-k", "opt175b-v"]), ("attn-out", ["opt175b-out"]),
                ("fc1", ["opt175b-fc1"]), ("fc2", ["opt175b-fc2"])]


class BlockGroup:
    """One input X, its Hessian and factor, and the layers quantized with them."""

    def __init__(self, label, names, dev, factor="R"):
        self.label = label
        self.factor = factor
        self.cfgs = [S.CONFIGS[n] for n in names]
        c0 = self.cfgs[0]
        d = c0.d
        self.x = S.make_activations(c0, dev)
        self.ws = [S.make_weights(c, dev) for c in self.cfgs]
        self.H = torch.empty(d, d, dtype=torch.float64, device=dev)
        self.U = torch.empty(d, d, dtype=torch.float64 if factor == "R" else torch.float32, device=dev)
        self.ws_h = torch.empty(max(1, G.workspace_bytes(G.WS_ACCUMULATE_HESSIAN, 0, d, c0.n_tokens)),
                                dtype=torch.uint8, device=dev)
        self.ws_c = torch.empty(G.workspace_bytes(G.WS_PREPARE_HINV, 0, d), dtype=torch.uint8, device=dev)
        qb = max(G.workspace_bytes(G.WS_QUANTIZE_LAYER, c.m, d, 0, G.make_qcfg(c.bits, c.group, c.grid, factor=factor))
                 for c in self.cfgs)
        self.ws_q = torch.empty(qb, dtype=torch.uint8, device=dev)
        self.outs = []
        for c in self.cfgs:
            ng = d // c.group if c.group else 1
            self.outs.append({
                "qcodes": torch.empty(c.m, d * c.bits // 32, dtype=torch.int32, device=dev),
                "scales": torch.empty(c.m, ng, dtype=torch.float32, device=dev),
                "zeros": torch.empty(c.m, ng, dtype=torch.uint8, device=dev),
                "w_hat": torch.empty(c.m, d, dtype=torch.float32, device=dev),
                "err_sq": torch.empty(c.m, dtype=torch.float32, device=dev)})
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 + len(self.cfgs))]

    def step(self):
        c0 = self.cfgs[0]
        self.ev[0].record()
        G.accumulate_hessian(self.H, self.x, accumulate=False, workspace=self.ws_h)
        self.ev[1].record()
        if self.factor == "R":
            _, self.info, _ = G.prepare_hchol(self.H, c0.damp, R=self.U, workspace=self.ws_c)
        else:
            _, self.info, _ = G.prepare_hinv(self.H, c0.damp, U=self.U, workspace=self.ws_c)
        self.ev[2].record()
        for i, (c, w, o) in enumerate(zip(self.cfgs, self.ws, self.outs)):
            G.quantize_layer(w, self.U, c.bits, c.group, c.grid, workspace=self.ws_q, out=o, factor=self.factor)
            self.ev[3 + i].record()

    def stage_ms(self):
        st = {"hessian": self.ev[0].elapsed_time(self.ev[1]), "hinv_chain": self.ev[1].elapsed_time(self.ev[2])}
        for i, c in enumerate(self.cfgs):
            st["quantize " + c.name] = self.ev[2 + i].elapsed_time(self.ev[3 + i])
        return st


def sequential_block_bench(args):
    """One step = the OPT-175B block quantized sublayer by sublayer, each on the
    calibration input the block's forward pass produces through the sublayers
    quantized before it (q, k, v on LN1(x); out on the attention output; fc1 on
    LN2(h); fc2 on ReLU(fc1)). The forward passes (torch) and the library's
    quantization are timed apart with HIP events."""
    from post_weight_quantization_18_amd import opt_block as B
    dev = torch.device("cuda:0")
    shape = B.OPT175B
    _say("sequential block: drawing the block input and the six weight matrices")
    x = B.block_input(shape, dev)
    sb = B.SequentialBlock(shape, dev, factor="U" if args.factor == "U" else "R")
    torch.cuda.synchronize()
    for i in range(args.warmup):
        sb.run(x)
        _say(f"sequential block warmup {i + 1}/{args.warmup} done: {sb.stage_s}")
    fwd, quant = 0.0, {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        sb.run(x)
        fwd += sb.stage_s["forward_ms"]
        for k, v in sb.stage_s["quantize_ms"].items():
            quant[k] = quant.get(k, 0.0) + v
        _say(f"sequential block step done: {sb.stage_s}")
    wall = time.perf_counter() - t0
    s_block = wall / args.steps
    n_weights = sum(c.n_weights for c in sb.cfgs.values())
    result = {
        "metric": "OPT-175B block quantization time, sublayers calibrated sequentially (one GPU, forward passes "
                  "included)",
        "value": s_block, "unit": "s/block", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(s_block * 1e3, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 MFMA->f32/f64 (H), f64 (R), f32 (column loop), split-f16 MFMA->f32 (trailing GEMM); "
                 "forward f16 products, f32 attention",
        "data": "synthetic block input (correlated Gaussian, 128 sequences of 2048 tokens) and synthetic weights",
        "config": {"workload": "OPT-175B decoder block: q, k, v, out 12288x12288, fc1 49152x12288, fc2 12288x49152; "
                               "3-bit asym g128; each sublayer calibrated on the forward pass through the quantized "
                               "sublayers before it; 262144 tokens", "weights": n_weights, "factor": sb.factor},
        "weights_per_s": n_weights / s_block,
        "forward_ms": round(fwd / args.steps, 3),
        "quantize_ms": {k: round(v / args.steps, 3) for k, v in quant.items()},
    }
    print(json.dumps(result), flush=True)


def block_bench(args):
    if args.sequential:
        sequential_block_bench(args)
        return
    dev = torch.device("cuda:0")
    groups = []
    for label, names in BLOCK_GROUPS:
        _say(f"block: drawing {label} ({', '.join(names)})")
        groups.append(BlockGroup(label, names, dev, factor="U" if args.factor == "U" else "R"))
    torch.cuda.synchronize()
    for i in range(args.warmup):
        for g in groups:
            g.step()
        torch.cuda.synchronize()
        _say(f"block warmup step {i + 1}/{args.warmup} done")
    if any(int(g.info.item()) != 0 for g in groups):
        raise RuntimeError("H + lambda I not positive definite")
    acc = {g.label: {} for g in groups}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for g in groups:
            g.step()
        torch.cuda.synchronize()
        for g in groups:
            for k, v in g.stage_ms().items():
                acc[g.label][k] = acc[g.label].get(k, 0.0) + v
        _say("block timed step done")
    wall = time.perf_counter() - t0
    s_block = wall / args.steps
    n_weights = sum(c.n_weights for g in groups for c in g.cfgs)
    result = {
        "metric": "OPT-175B block quantization time (one GPU, whole hot path for the block's six layers)",
        "value": s_block,
        "unit": "s/block",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(s_block * 1e3, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 MFMA->f32/f64 (H), f64 (R or U), f32 (column loop), split-f16 MFMA->f32 (trailing GEMM)",
        "data": "synthetic (seeded inputs and weights of the block's shapes; q, k and v share one input)",
        "config": {"workload": "OPT-175B block: q, k, v, out 12288x12288, fc1 49152x12288, fc2 12288x49152; "
                               "3-bit asym g128; 262144 calibration tokens per input; q/k/v share one H and factor",
                   "weights": n_weights, "factor": groups[0].factor},
        "weights_per_s": n_weights / s_block,
        "stages_ms": {g.label: {k: round(v / args.steps, 3) for k, v in acc[g.label].items()} for g in groups},
        "model_projection_96_blocks_min": round(96 * s_block / 60, 2),
    }
    print(json.dumps(result), flush=True)


def gemv_cpu_baseline(layers, rows=32):
    """The oracle's dequant_matvec on `rows` rows of each block layer (the same
    packed codes), scaled by m / rows per layer."""
    import oracle as O
    total, measured = 0.0, 0.0
    for name, q, sc, z, bits, group, x, y, nb, perm in layers:
        m = q.shape[0]
        qs = q[:rows].cpu().numpy().view(np.uint32)
        ss, zs, xs = sc[:rows].cpu().numpy(), z[:rows].cpu().numpy(), x.cpu().numpy()
        if perm is not None:
            xs = xs[perm[0].cpu().numpy()]  # act-order: the codes are in group order, x gathered to match
        t0 = time.perf_counter()
        O.dequant_matvec(qs, ss, zs, bits, group, xs)
        dt = time.perf_counter() - t0
        measured += dt
        total += dt * m / rows
    return {"value": 1.0 / total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"dequant_matvec on {rows} rows of each of the 6 layers, scaled by m/{rows}; measured "
                      f"{measured:.1f} s, extrapolated {total:.1f} s per token",
            "cpu": platform.processor() or platform.machine()}


def main():
    args = parse()
    if args.vendor_gemm:
        vendor_gemm()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.static_groups and not args.act_order:
        print("--static-groups needs --act-order", file=sys.stderr)
        sys.exit(2)
    if args.gemv:
        G.load_library()
        gemv_bench(args)
        return
    if args.block:
        G.load_library()
        block_bench(args)
        return
    cfg = S.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    G.load_library()
    _say(f"{cfg.name}: drawing W {cfg.m}x{cfg.d} and X {cfg.n_tokens}x{cfg.d}")
    w = S.make_weights(cfg, dev)
    x = S.make_activations(cfg, dev)
    torch.cuda.synchronize()
    _say("inputs resident; allocating buffers")
    factor = args.factor
    if factor == "auto":
        factor = "R" if cfg.d >= 8192 else "U"
    if factor == "R" and cfg.group > 128 and not (args.act_order and args.static_groups):
        factor = "U"  # groups wider than a block are refitted in the U form only
    run = LayerRun(cfg, w, x, args.chunk_tokens, args.act_order, args.static_groups, factor)
    for i in range(args.warmup):
        run.step()
        torch.cuda.synchronize()
        _say(f"warmup step {i + 1}/{args.warmup} done (untraced): {run.stage_ms()}")
    torch.cuda.synchronize()
    if run.info is not None and int(run.info.item()) != 0:
        raise RuntimeError("H + lambda I not positive definite")

    stage_acc = {}
    syrk_calls = []
    fam = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if not args.no_trace:
            G.trace_start()
        run.step(timed_chunks=True)
        torch.cuda.synchronize()
        if not args.no_trace:
            for k, v in G.trace_stop().items():
                f = fam.setdefault(k, {"launches": 0, "ms": 0.0, "work": 0.0})
                for q in f:
                    f[q] += v[q]
        for k, v in run.stage_ms().items():
            stage_acc[k] = stage_acc.get(k, 0.0) + v
        syrk_calls += run.syrk_call_ms()
        _say(f"timed step done: {run.stage_ms()}")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = {k: v / args.steps for k, v in stage_acc.items()}
    ms_per_step = wall * 1e3 / args.steps

    d, m, n = cfg.d, cfg.m, cfg.n_tokens
    # algorithmic work
    f_syrk_call = run.chunk * d * (d + 1)                     # lower triangle of 2 X^T X per call
    f_syrk = n * d * (d + 1)
    f_chain = (d ** 3 / 3 if run.factor == "R" else 2 * d ** 3 / 3)  # Cholesky (+ triangular inverse for U)
    f_trail = m * d * max(d - 128, 0)                            # W[:, later] -= E U[blk, later], every block
    f_loop = m * d * 128                                         # in-block updates (m d B)
    syrk_call_ms = sum(syrk_calls) / len(syrk_calls)
    syrk_tflops = f_syrk_call / (syrk_call_ms * 1e-3) / 1e12
    traffic = syrk_traffic(cfg.name, run.chunk)
    kernels = {}
    if fam:
        per = {k: {"launches": v["launches"] / args.steps, "ms": v["ms"] / args.steps, "work": v["work"] / args.steps}
               for k, v in fam.items()}

        def frac(flops, ms, peak):
            return None if not ms else round(flops / (ms * 1e-3) / 1e12 / peak, 4)
        sy = per.get("syrk", {"launches": 0, "ms": 0.0, "work": 0.0})
        tg = per.get("tgemm", {"launches": 0, "ms": 0.0, "work": 0.0})
        chain_ms = sum(v["ms"] for k, v in per.items() if k.startswith("chain_"))
        cl = per.get("colloop", {"launches": 0, "ms": 0.0, "work": 0.0})
        # per launch of the SYRK: the tokens of one launch (the library cuts long calls into launches)
        sy_tokens = n / sy["launches"] if sy["launches"] else 0
        kernels = {
            "syrk_kernel": {"bound": "mfma fp16", "launches": sy["launches"], "ms": round(sy["ms"], 3),
                            "avg_ms": round(sy["ms"] / max(sy["launches"], 1), 4),
                            "algorithmic_tflops": round(f_syrk / (sy["ms"] * 1e-3) / 1e12, 2) if sy["ms"] else None,
                            "frac_algorithmic": frac(f_syrk, sy["ms"], PEAK_FP16_TFLOPS),
                            "frac_executed": frac(sy["work"], sy["ms"], PEAK_FP16_TFLOPS),
                            "tokens_per_launch": sy_tokens},
            "tgemm_kernel": {"bound": "mfma fp16 (three split-fp16 passes)", "launches": tg["launches"],
                             "ms": round(tg["ms"], 3),
                             "algorithmic_tflops": round(f_trail / (tg["ms"] * 1e-3) / 1e12, 2) if tg["ms"] else None,
                             "frac_algorithmic": frac(f_trail, tg["ms"], PEAK_FP16_TFLOPS),
                             "frac_executed": frac(tg["work"], tg["ms"], PEAK_FP16_TFLOPS)},
            "chain_fp64": {"bound": "mfma fp64", "ms": round(chain_ms, 3),
                           "launches": sum(v["launches"] for k, v in per.items() if k.startswith("chain_")),
                           "flops": ("d^3 / 3 (Cholesky of H_d; R form)" if run.factor == "R"
                                     else "2 d^3 / 3 (Cholesky + triangular inverse)"),
                           "frac": frac(f_chain, chain_ms, PEAK_FP64_TFLOPS),
                           "by_family_ms": {k: round(v["ms"], 3) for k, v in per.items() if k.startswith("chain_")}},
            "colloop_kernel": {"bound": "alu fp32 / LDS (d dependent steps)", "launches": cl["launches"],
                               "ms": round(cl["ms"], 3),
                               "frac_fp32_vector": frac(f_loop, cl["ms"], PEAK_FP32_VECTOR_TFLOPS)},
            "other_ms": {k: round(v["ms"], 3) for k, v in per.items()
                         if k not in ("syrk", "tgemm", "colloop") and not k.startswith("chain_")},
        }
        if sy["launches"]:
            # the roofline is taken per launch of the SYRK kernel itself (the split-K combine is listed apart)
            syrk_call_ms = sy["ms"] / sy["launches"]
            f_syrk_call = sy_tokens * d * (d + 1)
            syrk_tflops = f_syrk_call / (syrk_call_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "syrk_kernel (Hessian SYRK, fp16 MFMA, fp32 accumulate)",
                "achieved": round(syrk_tflops, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(syrk_tflops / PEAK_FP16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "traffic_unit": "HBM bytes per syrk_kernel launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                "per_launch": {"flops": f_syrk_call, "avg_ms": round(syrk_call_ms, 4)}}
    result = {
        "metric": "GPTQ layer quantize throughput (weights quantized per second, whole hot path)",
        "value": cfg.n_weights / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA->f32/f64 (H), f64 (R or U), f32 (column loop), split-f16 MFMA->f32 (trailing GEMM)",
        "data": "synthetic (seeded correlated-Gaussian X with outlier channels, N(0,0.02^2) W with outlier columns)",
        "config": {"workload": f"{cfg.name}: W {m}x{d} {cfg.w_dtype}, X {n}x{d} fp16, {cfg.bits}-bit {cfg.grid} "
                               f"{'per-row' if cfg.group == 0 else 'g' + str(cfg.group)}, block 128, damp {cfg.damp}"
                               + (", act-order" + (" + static groups" if args.static_groups else "")
                                  if args.act_order else ""),
                   "chunk_tokens": run.chunk, "m": m, "d": d, "n_tokens": n,
                   "factor": ("R (Cholesky factor of H_d, gptq_prepare_hchol)" if run.factor == "R"
                              else "U (chol(H_d^-1), gptq_prepare_hinv)")},
        "layer_time_s": round(ms_per_step * 1e-3, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage.items()},
        "mfma_frac": {"syrk_fp16": round(f_syrk / (stage["hessian"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                      "chain_fp64": round(f_chain / (stage["hinv_chain"] * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4)},
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        _say("timing the oracle on a bounded sample (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(cfg, w, x, args.cpu_sample_rows, args.cpu_sample_tokens,
                                              args.act_order, args.static_groups)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
