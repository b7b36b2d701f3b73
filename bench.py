#!/usr/bin/env python3
"""Decode benchmark of the activation-sparse FFN path on one MI355X.

Workload: the Llama3.2-3B-shaped 28-layer SwiGLU FFN stack (d_model 3072,
d_ff 8192, bf16 N(0, 0.02^2) weights, seed 0) run the SelectInfer way:
static base set = top 20% of neurons by Eq (1) over 512 calibration
tokens, dynamic set = top 20% by frequency of per-token top-30% over a
256-token prompt, unioned; then decode at batch 1 over the union.

A step is one decode token through all 28 layers (per layer: the gathered
gate/up activations over U_l, then the gathered down product accumulated
into the residual).  Calibration and prefill run once before timing (their
times are reported under "setup").  The timed steps replay a HIP graph of
one step; inputs (weights, index sets, tokens) are resident in HBM.

Reported: "value" = decode us/token (lower is better); "roofline" for the
dominant kernel (gathered gate/up) from per-launch HIP events; and
"cpu_baseline" = the CPU oracle on a bounded sample of the same decode.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
COPY_CALIB_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_rowop_glu_c1.json")


def measured_traffic(kernel_sources):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current source of that kernel."""
    import hashlib
    import json as _json
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = _json.load(fh)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for path in kernel_sources:
        with open(path, "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="bounded CPU work for the oracle baseline (0 disables it)")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def glu_bytes(u: int, d: int) -> int:
    """Algorithmic bytes of one gate/up launch over the u compacted neurons:
    2 bf16 rows of d per neuron, the input h read, the fp32 activations
    written."""
    return 2 * u * d * 2 + 4 * d + 4 * u


def down_bytes(u: int, d: int) -> int:
    """Down product over the compacted neurons: d output rows of u bf16
    weights, the activations read, the residual read and written."""
    return u * d * 2 + 4 * u + 2 * 4 * d


def cpu_baseline(layers, U_sets, X, seconds: float, rms_eps: float):
    """Time the CPU oracle's decode of whole tokens through the stack until
    ``seconds`` of work are done (at least one token)."""
    import oracle
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        pass
    t0 = time.perf_counter()
    tokens = 0
    while True:
        h = X[tokens % X.shape[0]].astype(np.float64)
        for l, (Wg, Wu, WdT) in enumerate(layers):
            _, y = oracle.decode_over_set(Wg, Wu, WdT, oracle.rms_normalize(h, rms_eps), U_sets[l])
            h = h + y
        tokens += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=dt / tokens * 1e6, unit="us/token", cores=threads or os.cpu_count(),
                kind="oracle",
                sample=f"{tokens} decode token(s) x 28 layers over the same union sets, "
                       f"numpy fp64, {dt:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    from activation_sparse_decode_amd import binding as B
    from activation_sparse_decode_amd import synth
    from activation_sparse_decode_amd.pipelines import (RMS_EPS, SelectInferStack, pct_count,
                                                        to_device_bf16)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()

    cfg = synth.SHAPES["c1"]
    L, N, d = cfg["layers"], cfg["n"], cfg["d"]
    t0 = time.perf_counter()
    threads = min(16, os.cpu_count() or 1)
    layers = synth.ffn_stack(args.seed, synth.W_C1, L, N, d, threads=threads)
    dev_layers = [tuple(to_device_bf16(m, dev) for m in lay) for lay in layers]
    log(f"weights: {L} layers x 3 x [{N} x {d}] bf16 in {time.perf_counter() - t0:.1f} s")

    base_k = pct_count(cfg["base_pct"], N)
    alpha_k = pct_count(cfg["alpha_pct"], N)
    beta_k = pct_count(cfg["beta_pct"], N)
    stack = SelectInferStack(dev_layers, base_k, alpha_k, beta_k,
                             max_tokens=max(cfg["calib_tokens"], cfg["prompt_tokens"]))
    Xc = torch.from_numpy(synth.tokens(args.seed, synth.W_C1, 1, cfg["calib_tokens"], d)).to(dev)
    Xp = torch.from_numpy(synth.tokens(args.seed, synth.W_C1, 2, cfg["prompt_tokens"], d)).to(dev)
    n_tok = args.warmup + args.steps
    Xd_host = synth.tokens(args.seed, synth.W_C1, 3, n_tok, d)
    Xd = torch.from_numpy(Xd_host).to(dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    e0, e1, e2 = ev(), ev(), ev()
    torch.cuda.synchronize()
    e0.record()
    stack.calibrate(Xc)
    e1.record()
    stack.prefill(Xp)
    e2.record()
    torch.cuda.synchronize()
    calib_ms, prefill_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    U_cnt = stack.U_cnt.cpu().numpy().astype(np.int64)
    log(f"calibration {calib_ms:.1f} ms, prefill {prefill_ms:.1f} ms; |U| mean {U_cnt.mean():.0f}")

    step_bytes = int(sum(glu_bytes(u, d) + down_bytes(u, d) for u in U_cnt))
    glu_total_bytes = int(sum(glu_bytes(u, d) for u in U_cnt))

    # ---- one decode step captured as a HIP graph
    h = torch.zeros(d, dtype=torch.float32, device=dev)
    xcur = torch.zeros(d, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.copy_(xcur)
        stack.decode(h)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h.copy_(xcur)
        stack.decode(h)
    torch.cuda.synchronize()

    for t in range(args.warmup):
        xcur.copy_(Xd[t])
        graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: K graph-replayed decode steps
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record()
    for t in range(args.warmup, n_tok):
        xcur.copy_(Xd[t])
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    us_per_token = total_ms * 1e3 / args.steps
    log(f"decode: {us_per_token:.1f} us/token over {args.steps} steps")

    # ---- dominant kernel (gate/up over the compacted union): its 28
    # launches of one decode step captured alone in a graph and replayed K
    # times on the same stream, bracketed by HIP events (per-launch events
    # in eager mode would add their own overhead to every short launch).
    glu_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(glu_graph):
        for l in range(L):
            stack.decode_gate_up(l, h)
    torch.cuda.synchronize()
    for _ in range(2):
        glu_graph.replay()
    g0, g1 = ev(), ev()
    torch.cuda.synchronize()
    g0.record()
    for _ in range(args.steps):
        glu_graph.replay()
    g1.record()
    torch.cuda.synchronize()
    glu_us = g0.elapsed_time(g1) * 1e3 / (args.steps * L)
    achieved = glu_total_bytes / L / (glu_us * 1e-6) / 1e9
    log(f"gate/up over U: {glu_us:.2f} us/launch avg, {achieved:.0f} GB/s")

    # A plain device copy of known size: the reference that scales the HBM
    # counters (FETCH_SIZE / WRITE_SIZE) of the profiled kernels to bytes.
    calib = torch.empty(COPY_CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    torch.cuda.synchronize()

    cpu = None
    if args.cpu_seconds > 0:
        U_sets = [stack.U_idx[l, :U_cnt[l]].cpu().numpy() for l in range(L)]
        cpu = cpu_baseline(layers, U_sets, Xd_host, args.cpu_seconds, RMS_EPS)
        log(f"cpu oracle: {cpu['value']:.0f} us/token on {cpu['cores']} threads")

    out = {
        "metric": "sparse-FFN decode us/token and achieved HBM GB/s (% of peak) at batch 1",
        "value": round(us_per_token, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "weight_dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) bf16 weights, heavy-tailed tokens; no trained weights)",
        "config": {
            "workload": "SelectInfer 28-layer FFN stack, Llama3.2-3B shape (d_model 3072, d_ff 8192), "
                        "base 20% by Eq (1) over 512 calibration tokens, per-token top-30% / "
                        "frequency top-20% over a 256-token prompt, union; decode at batch 1",
            "layers": L, "d_model": d, "d_ff": N, "batch": 1,
            "union_mean": round(float(U_cnt.mean()), 1), "union_min": int(U_cnt.min()),
            "union_max": int(U_cnt.max()),
        },
        "step_bytes": step_bytes,
        "step_GBps": round(step_bytes / (us_per_token * 1e-6) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (us_per_token * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "setup": {"calibrate_ms": round(calib_ms, 2), "prefill_ms": round(prefill_ms, 2)},
        "roofline": {
            "kernel": "rowop_b1_kernel<GLU> (gate/up over the compacted union, SwiGLU epilogue)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic([
                os.path.join(ROOT, "activation_sparse_decode_amd", "csrc", "rowop_b1.hip"),
                os.path.join(ROOT, "activation_sparse_decode_amd", "csrc", "sffn_device.h")]),
            "launch_us": round(glu_us, 3),
            "bytes_per_launch": int(glu_total_bytes / L),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
