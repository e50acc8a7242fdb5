"""Per-layer run of an OPT block's six layers through the library, with resume
and one JSON line per (config, layer).

    python tests/block_parity_harness.py --out DIR [--resume] [--layers q,k,v,out,fc1,fc2]
                                         [--rows N] [--parity-max-d D] [--tokens N]

Each layer is quantized on cuda:0 from its synthetic W and X (the q, k and v
layers share one input, so one Hessian and one factor serve the three). Its
packed codes, scales, zero points and error sums go to DIR/<layer>.npz, and a
JSON line goes to DIR/results.jsonl and to stdout with:
  * stage times (HIP events around the Hessian, the factor and the quantizer),
  * algorithmic flops and bytes of the layer, the SYRK's and the chain's
    fraction of the matrix-core peak, and weights per second;
  * parity on sampled rows against the oracle (its own fp64 H over all tokens,
    lambda and factor, follow mode and a free run), the oracle's time and the
    host's core count, or why parity was skipped (the oracle's H at d = 49152
    would take about 20 minutes of host time).
With --resume, layers that already have their .npz and a line in
results.jsonl are skipped, so an interrupted run continues at the next layer.

This is test infrastructure: it calls the oracle, and nothing in the library
imports it.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

from post_weight_quantization_18_amd import gptq as G  # noqa: E402
from post_weight_quantization_18_amd import synthetic as S  # noqa: E402

BLOCK = "opt175b-block"
LAYERS = {"q": "opt175b-q", "k": "opt175b-k", "v": "opt175b-v", "out": "opt175b-out",
          "fc1": "opt175b-fc1", "fc2": "opt175b-fc2"}
SHARED = [["q", "k", "v"], ["out"], ["fc1"], ["fc2"]]   # layers that read one input
PEAK_FP16_TFLOPS = 2516.6
PEAK_FP64_TFLOPS = 78.6


def completed(out_dir):
    """Layers with a results line and their .npz in out_dir."""
    path = os.path.join(out_dir, "results.jsonl")
    done = set()
    if os.path.exists(path):
        for line in open(path):
            line = line.strip()
            if not line:
                continue
            rec = json.loads(line)
            if rec.get("config") == BLOCK and os.path.exists(os.path.join(out_dir, rec["layer"] + ".npz")):
                done.add(rec["layer"])
    return done


def plan(layers, done):
    """The shared-input groups still to run, each with the layers it must
    quantize (a group is skipped only when all its requested layers are done)."""
    todo = []
    for group in SHARED:
        want = [l for l in group if l in layers and l not in done]
        if want:
            todo.append((group, want))
    return todo


def layer_work(cfg, n_tokens=None):
    """Algorithmic flops and bytes of one layer (the R factor: no inverse)."""
    m, d, n = cfg.m, cfg.d, n_tokens or cfg.n_tokens
    flops = {"syrk": n * d * (d + 1), "chain": d ** 3 / 3, "trailing": m * d * max(d - 128, 0),
             "column_loop": m * d * 128}
    nbytes = {"x": 2 * n * d, "w": 2 * m * d, "h": 8 * d * d, "r": 8 * d * d,
              "outputs": m * d * cfg.bits // 8 + m * (d // cfg.group if cfg.group else 1) * 5 + 4 * m}
    return flops, nbytes


def write_record(out_dir, rec):
    line = json.dumps(rec)
    with open(os.path.join(out_dir, "results.jsonl"), "a") as fh:
        fh.write(line + "\n")
    print(line, flush=True)


def upper_inverse(r, leaf=4096, say=None):
    """The inverse of the upper triangular r by halves: [[A, B], [0, C]]^-1 =
    [[A^-1, -A^-1 B C^-1], [0, C^-1]], leaves of at most `leaf` columns by a
    triangular solve. Only general matrix products of explicit copies touch
    the whole width (the BLAS routines for symmetric or triangular operands
    are not trusted with arrays of 2^31 entries)."""
    import scipy.linalg as sl
    n = r.shape[0]
    if n <= leaf:
        return sl.solve_triangular(r, np.eye(n), lower=False)
    k = max(leaf, (n // 2) // leaf * leaf)
    ai = upper_inverse(r[:k, :k], leaf, say)
    ci = upper_inverse(r[k:, k:], leaf, say)
    out = np.zeros((n, n))
    out[:k, :k] = ai
    out[k:, k:] = ci
    out[:k, k:] = -(ai @ np.ascontiguousarray(r[:k, k:])) @ ci
    if say is not None:
        say(f"[harness] oracle U = R^-1: block of {n} columns done")
    return out


def _print_line(text):
    print(text, flush=True)


def oracle_factor_in_steps(xh, damp, chunk=4096, log=_print_line):
    """The oracle's H over the tokens chunk by chunk (each chunk's 2 X_c^T X_c
    summed in order, which is exactly the oracle's own sum), lambda, its R =
    hessian_factor(H_d) (a line per column block), and U = R^-1 (pinned in
    the oracle's tests) by halves. Every step prints a line, so that the
    longest silent step is one chunk or one block (log: where the lines go)."""
    import oracle as O
    n, d = xh.shape
    h = None
    for t0 in range(0, n, chunk):
        part = O.hessian(xh[t0:t0 + chunk])
        if h is None:
            h = part
        else:
            h += part  # the oracle's sum over chunks, in place
        del part
        log(f"[harness] oracle H: {min(t0 + chunk, n)} / {n} tokens")
    hd, lam = O.damp(h, damp)
    r = O.hessian_factor(hd, progress=lambda k, dd: log(f"[harness] oracle R: {k} / {dd} columns"))
    log("[harness] oracle R = hessian_factor(H_d) done")
    u = upper_inverse(r, say=log)  # upper triangular by construction
    log("[harness] oracle U = R^-1 done")
    return h, lam, u, hd, r


def compare_rows_in_steps(wn, gpu, oracle, bits, group, grid, label, log=_print_line):
    """compare_rows for wide layers, a line after each step (the factor
    statistics, the oracle's follow mode, its free run)."""
    import oracle as O
    from parity_util import _factor_stats, _row_stats
    h, lam, u, hd, r = oracle
    t0 = time.time()
    stats = {"label": label, "rows": wn.shape[0]}
    _factor_stats(stats, gpu, h, lam, u, hd, r_oracle=r)
    log(f"[harness] {label}: factor statistics done")
    follow = O.gptq_quantize(wn, u, bits, grid, group, follow_codes=gpu["codes"], follow_zeros=gpu["zeros"])
    log(f"[harness] {label}: oracle follow mode done")
    free = O.gptq_quantize(wn, u, bits, grid, group)
    log(f"[harness] {label}: oracle free run done")
    _row_stats(stats, wn, gpu, follow, free, h, bits, grid, group)
    stats["oracle_s"] = time.time() - t0
    return stats


def run_group(group, want, out_dir, n_rows, parity_max_d, dev, tokens=0):
    import oracle as O  # noqa: F401  (test infrastructure only)
    from parity_util import compare_rows, device_factor_r, failed_gates, oracle_factor, rows_of, sample_rows

    cfgs = {l: S.CONFIGS[LAYERS[l]] for l in group}
    c0 = cfgs[group[0]]
    print(f"[harness] {group}: drawing X ({c0.n_tokens} x {c0.d}) and W", flush=True)
    x = S.make_activations(c0, dev)
    if tokens:
        x = x[:tokens].contiguous()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    H = torch.empty(c0.d, c0.d, dtype=torch.float64, device=dev)
    G.accumulate_hessian(H, x, accumulate=False)
    ev[1].record()
    R, info, lam = G.prepare_hchol(H, c0.damp, r_dtype=torch.float64)
    ev[2].record()
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        raise RuntimeError(f"H + lambda I of {group} is not positive definite (info {int(info.item())})")
    h_ms, f_ms = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    lam = float(lam.item())
    parity_ok = c0.d <= parity_max_d
    oracle = None
    results = {}
    for l in want:
        cfg = cfgs[l]
        w = S.make_weights(cfg, dev)
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        res = G.quantize_layer(w, R, cfg.bits, cfg.group, cfg.grid, factor="R")
        q1.record()
        torch.cuda.synchronize()
        q_ms = q0.elapsed_time(q1)
        np.savez(os.path.join(out_dir, l + ".npz"), qcodes=res["qcodes"].cpu().numpy().view(np.uint32),
                 scales=res["scales"].cpu().numpy(), zeros=res["zeros"].cpu().numpy(),
                 err_sq=res["err_sq"].cpu().numpy())
        rows = sample_rows(cfg.m, 21 + cfg.layer_id, n_rows)
        results[l] = (cfg, q_ms, rows_of(res, rows, cfg.bits, cfg.d), rows,
                      w[torch.as_tensor(rows, device=dev)].double().cpu().numpy())
        del res, w
    factor = {"H": H.cpu().numpy(), "U": R.cpu().double().numpy(), "lam": lam, "u_eps": 2.0 ** -53, "factor": "R"}
    xh = x.cpu().numpy() if parity_ok else None
    del H, R, x
    torch.cuda.empty_cache()
    t_or = time.time()
    if parity_ok:
        print(f"[harness] {group}: oracle H, lambda and factor over {xh.shape[0]} tokens", flush=True)
        oracle = oracle_factor(xh, c0.damp) if c0.d <= 12288 else oracle_factor_in_steps(xh, c0.damp)
        del xh
    oracle_factor_s = time.time() - t_or
    for i, l in enumerate(want):
        cfg, q_ms, gr, rows, wn = results[l]
        flops, nbytes = layer_work(cfg, tokens or cfg.n_tokens)
        # the shared Hessian and factor are charged to the first layer of the group
        hh, ff = (h_ms, f_ms) if i == 0 else (0.0, 0.0)
        total = hh + ff + q_ms
        rec = {"config": BLOCK, "layer": l, "workload": cfg.name, "m": cfg.m, "d": cfg.d,
               "n_tokens": tokens or cfg.n_tokens,
               "bits": cfg.bits, "group": cfg.group, "grid": cfg.grid, "factor": "R",
               "shared_input": group, "stage_ms": {"hessian": round(hh, 3), "factor": round(ff, 3),
                                                   "quantize": round(q_ms, 3), "total": round(total, 3)},
               "flops": flops, "bytes": nbytes,
               "mfma_frac": {"syrk_fp16": round(flops["syrk"] / (h_ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                             "chain_fp64": round(flops["chain"] / (f_ms * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4)},
               "weights_per_s": cfg.m * cfg.d / (total * 1e-3),
               "host_cores": len(os.sched_getaffinity(0)), "torch_threads": torch.get_num_threads()}
        if parity_ok:
            h, lam_o, u, hd = oracle[:4]
            gr.update(factor)
            t1 = time.time()
            label = f"{cfg.name} ({len(rows)} rows)"
            if len(oracle) == 5:
                stats = compare_rows_in_steps(wn, gr, oracle, cfg.bits, cfg.group, cfg.grid, label)
            else:
                stats = compare_rows(wn, gr, h, lam_o, u, hd, cfg.bits, cfg.group, cfg.grid, label)
            failed = failed_gates(stats)  # reported, not raised: the line records the failure
            gates = "pass" if not failed else "fail: " + ", ".join(failed)
            rec["parity"] = {k: (float(v) if isinstance(v, (np.floating, float)) else v) for k, v in stats.items()
                             if isinstance(v, (int, float, bool, str, np.floating, np.integer))}
            # (row, column) of the first hard mismatches, if any
            rec["parity"]["hard_at"] = [[int(r), int(j)] for r, j in stats.get("hard_at", [])]
            rec["parity"]["gates"] = gates
            rec["oracle_s"] = round(oracle_factor_s + (time.time() - t1), 1)
        else:
            rec["parity"] = {"skipped": f"the oracle's H at d = {cfg.d} over {cfg.n_tokens} tokens "
                                        f"({2 * cfg.n_tokens * cfg.d ** 2 / 2:.1e} fp64 flops on the host) exceeds "
                                        f"--parity-max-d {parity_max_d}"}
        write_record(out_dir, rec)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--resume", action="store_true")
    ap.add_argument("--layers", default=",".join(LAYERS))
    ap.add_argument("--rows", type=int, default=64, help="sampled rows per layer for parity")
    ap.add_argument("--parity-max-d", type=int, default=12288)
    ap.add_argument("--tokens", type=int, default=0,
                    help="calibrate on the first N tokens of each layer's X (0: all 262144); a stand-in that lets "
                         "the oracle's own H at d = 49152 fit the host's time")
    args = ap.parse_args(argv)
    layers = [l for l in args.layers.split(",") if l]
    for l in layers:
        if l not in LAYERS:
            raise SystemExit(f"unknown layer {l}; choose from {list(LAYERS)}")
    os.makedirs(args.out, exist_ok=True)
    done = completed(args.out) if args.resume else set()
    if not args.resume and os.path.exists(os.path.join(args.out, "results.jsonl")):
        os.remove(os.path.join(args.out, "results.jsonl"))
    todo = plan(layers, done)
    if done:
        print(f"[harness] resuming: done {sorted(done)}; to run {[w for _, w in todo]}", flush=True)
    dev = torch.device("cuda:0")
    G.load_library()
    for group, want in todo:
        run_group(group, want, args.out, args.rows, args.parity_max_d, dev, args.tokens)
    print("[harness] done", flush=True)


if __name__ == "__main__":
    main()
