#!/usr/bin/env python3
"""Decode benchmark of the activation-sparse FFN path on one MI355X.

Default workload (the one the headline metric is quoted on): the
Llama3.2-3B-shaped 28-layer SwiGLU FFN stack (d_model 3072, d_ff 8192, bf16
N(0, 0.02^2) weights, seed 0) run the SelectInfer way: static base set =
top 20% of neurons by Eq (1) over 512 calibration tokens, dynamic set = top
20% by frequency of per-token top-30% over a 256-token prompt, unioned; then
decode at batch 1 over the union.  A step is one decode token through all 28
layers (per layer: gate/up over U_l, then the down product over U_l added to
the residual).  Calibration, prefill and the per-prompt compaction run once
before timing (reported under "setup").

The default run (--workload all) reports that stack as the line's value and
adds every other workload under "configs", each with its own gathered
kernel as the roofline: c0 single layer with per-token top-50% (every step
runs activations, keys, select, compaction and the gathered down product),
c2 SpAx three-tier QKV + down read, c3 ReLU-sparse MoE stack (32 layers x 8
experts, top-2, 32-row clusters), c4 batched decode with a per-token
top-40% union contracted on MFMA at batch 1, 4, 8 and 16.  --workload runs
one of them alone (also c1-loading: the stack with SelectInfer's Table 1
knobs, and the --predictor / --weight-aware variants).

Every timed step is replayed from a HIP graph with its inputs resident in
HBM; the weights cycle through enough copies to exceed the 256 MB Infinity
Cache.  "roofline" is the workload's gathered (sparse) product: algorithmic
bytes per launch over its average launch time, the launches replayed alone
from a graph between HIP events on the stream they run on; the dense
kernels that feed a selection are reported beside it.  "cpu_baseline" is
the CPU oracle on a bounded sample of the same work, with all host cores
and with one.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
COPY_CALIB_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "activation_sparse_decode_amd", "csrc")
METRIC = "sparse-FFN decode us/token and achieved HBM GB/s (% of peak) at batch 1"
# sources of the gathered products (a committed traffic figure is reported
# only while they are unchanged)
AXPY_B1_SOURCES = ["axpy_b1.hip", "sffn_splitk.h", "sffn_device.h"]
AXPY_MFMA_SOURCES = ["axpy_mfma.hip", "axpy_b1.hip", "sffn_splitk.h", "sffn_device.h"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--workload", default="all",
                   choices=["all", "c0", "c1", "c1-loading", "c2", "c3", "c4"])
    p.add_argument("--batch", type=int, default=16, help="tokens per step of workload c4")
    p.add_argument("--layout", choices=("packed", "rows"), default="packed",
                   help="c4 at batch > 1: weights packed for the batched kernels, or row-major")
    p.add_argument("--union", choices=("mask", "list"), default="mask",
                   help="c4 at batch > 1: union formed in the product from the token masks, "
                        "or listed first (frequency counts and a union select)")
    p.add_argument("--predictor", action="store_true",
                   help="workload c3: clusters from an online predictor (PowerInfer-2), no dense gate")
    p.add_argument("--weight-aware", action="store_true",
                   help="workload c2: rank columns by |x_j| * ||W[:, j]||_2 (WiSparse)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="bounded CPU work for the oracle baseline, per thread setting "
                        "(0 disables it)")
    p.add_argument("--cpu-seconds-sub", type=float, default=2.5,
                   help="the same for each workload under \"configs\" of the default run")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return os.cpu_count()


def measured_traffic(tag: str, sources):
    """HBM bytes per launch of a dominant kernel from the committed counter
    summary profiles/traffic_<tag>.json, if it was taken on the current
    source of that kernel; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", f"traffic_{tag}.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """Graph capture and HIP-event timing on torch's current stream."""

    def __init__(self, torch):
        self.torch = torch

    def capture(self, body):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            body()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        torch.cuda.synchronize()
        return g

    def step_stats(self, graphs, reps, before=None, per_step=1):
        """Median, p10 and p90 of the per-replay time (us per unit of work), in
        a pass of its own with HIP events around every replay (the per-step
        input copies of before(i) fall outside the pairs).  `graphs` is one
        graph replayed `reps` times, or a list replayed in turn."""
        torch = self.torch
        seq = graphs if isinstance(graphs, (list, tuple)) else [graphs] * reps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in seq]
        for i, g in enumerate(seq):
            if before:
                before(i)
            ev[i][0].record()
            g.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) * 1e3 / per_step for a, b in ev])
        return {"median_us": round(float(np.median(t)), 3),
                "p10_us": round(float(np.percentile(t, 10)), 3),
                "p90_us": round(float(np.percentile(t, 90)), 3), "replays": len(seq)}

    def replay_ms(self, g, reps, before=None):
        """Total ms of `reps` replays (each optionally preceded by before(i))."""
        torch = self.torch
        for i in range(2):
            if before:
                before(i)
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            if before:
                before(i)
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)


def roofline(kernel, bytes_per_launch, launch_us, traffic=None):
    achieved = bytes_per_launch / (launch_us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "launch_us": round(launch_us, 3), "bytes_per_launch": int(bytes_per_launch)}


def result(value, unit, steps, warmup, ms_per_step, config, **extra):
    out = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "weight_dtype": "bf16",
           "data": "synthetic (seeded N(0,0.02^2) bf16 weights, heavy-tailed tokens; "
                   "no trained weights)",
           "config": config}
    out.update(extra)
    return out


def timed_cpu(fn, seconds, per_unit=1):
    """Run fn(i) until `seconds` of CPU work are done (at least once);
    returns (seconds per unit, count)."""
    t0, n = time.perf_counter(), 0
    while True:
        fn(n)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return (time.perf_counter() - t0) / (n * per_unit), n


def cpu_baseline(fn, seconds, sample, per_unit=1, scale=1e6, unit="us/token"):
    """The oracle on a bounded sample: timed with the BLAS pool at all host
    cores, then again limited to one thread.  value = seconds per unit x scale."""
    s_all, n_all = timed_cpu(fn, seconds, per_unit)
    cores = blas_threads()
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            s_one, n_one = timed_cpu(fn, seconds, per_unit)
        one = {"value": s_one * scale, "cores": 1, "sample_units": n_one}
    except ImportError:
        pass
    return {"value": s_all * scale, "unit": unit, "cores": cores, "host_cpus": os.cpu_count(),
            "kind": "oracle", "sample": f"{n_all} x {sample}", "one_core": one}


# ============================================================ c1: SelectInfer stack

def keyed_down_bytes(n: int, k: int, d: int) -> int:
    """Algorithmic bytes of one keyed batch-1 product: the k selected rows
    (d bf16 each), every neuron's 4-byte key, the k selected activations, the
    threshold pair and the d fp32 outputs written."""
    return k * d * 2 + 4 * n + 4 * k + 8 + 4 * d


def glu_bytes(u: int, d: int) -> int:
    """One gate/up launch over u compacted neurons: 2 bf16 rows of d per
    neuron, the input h read, the fp32 activations written."""
    return 2 * u * d * 2 + 4 * d + 4 * u


def down_bytes(u: int, d: int) -> int:
    """Down product over u compacted neurons: d output rows of u bf16
    weights, the activations read, the residual read and written."""
    return u * d * 2 + 4 * u + 2 * 4 * d


def run_c1(args, torch, B, synth, P, T):
    cfg = synth.SHAPES["c1"]
    L, N, d = cfg["layers"], cfg["n"], cfg["d"]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    layers = synth.ffn_stack(args.seed, synth.W_C1, L, N, d, threads=min(16, os.cpu_count() or 1))
    dev_layers = [tuple(P.to_device_bf16(m, dev) for m in lay) for lay in layers]
    log(f"weights: {L} layers x 3 x [{N} x {d}] bf16 in {time.perf_counter() - t0:.1f} s")
    stack = P.SelectInferStack(dev_layers, P.pct_count(cfg["base_pct"], N),
                               P.pct_count(cfg["alpha_pct"], N), P.pct_count(cfg["beta_pct"], N),
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
    stack.prefill(Xp)          # includes the per-prompt compaction
    e2.record()
    torch.cuda.synchronize()
    calib_ms, prefill_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    U_cnt = stack.U_cnt.cpu().numpy().astype(np.int64)
    log(f"calibration {calib_ms:.1f} ms, prefill + compaction {prefill_ms:.1f} ms; "
        f"|U| mean {U_cnt.mean():.0f}")
    step_bytes = int(sum(glu_bytes(u, d) + down_bytes(u, d) for u in U_cnt))
    glu_total = int(sum(glu_bytes(u, d) for u in U_cnt))

    h = torch.zeros(d, dtype=torch.float32, device=dev)
    xcur = torch.zeros(d, dtype=torch.float32, device=dev)

    def step():
        h.copy_(xcur)
        stack.decode(h)

    g = T.capture(step)
    for t in range(args.warmup):
        xcur.copy_(Xd[t])
        g.replay()
    torch.cuda.synchronize()
    total_ms = T.replay_ms(g, args.steps, before=lambda i: xcur.copy_(Xd[args.warmup + i]))
    us_tok = total_ms * 1e3 / args.steps
    log(f"decode: {us_tok:.1f} us/token over {args.steps} steps")
    dist = T.step_stats(g, args.steps, before=lambda i: xcur.copy_(Xd[args.warmup + i]))

    gg = T.capture(lambda: [stack.decode_gate_up(l, h) for l in range(L)])
    glu_us = T.replay_ms(gg, args.steps) * 1e3 / (args.steps * L)
    log(f"gate/up over U: {glu_us:.2f} us/launch")
    fused = run_c1_fused(args, torch, stack, Xd, h, xcur, g, L, d, U_cnt, T)

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        U_sets = [stack.U_idx[l, :U_cnt[l]].cpu().numpy() for l in range(L)]

        def one(i):
            hh = Xd_host[i % Xd_host.shape[0]].astype(np.float64)
            for l, (Wg, Wu, WdT) in enumerate(layers):
                _, y = oracle.decode_over_set(Wg, Wu, WdT, oracle.rms_normalize(hh, P.RMS_EPS),
                                              U_sets[l])
                hh = hh + y

        cpu = cpu_baseline(one, args.cpu_seconds,
                           "decode token(s) x 28 layers over the same union sets, numpy fp64")

    config = {"workload": "SelectInfer 28-layer FFN stack, Llama3.2-3B shape (d_model 3072, "
                          "d_ff 8192), base 20% by Eq (1) over 512 calibration tokens, per-token "
                          "top-30% / frequency top-20% over a 256-token prompt, union; decode at "
                          "batch 1 over the per-prompt compacted union",
              "layers": L, "d_model": d, "d_ff": N, "batch": 1,
              "union_mean": round(float(U_cnt.mean()), 1), "union_min": int(U_cnt.min()),
              "union_max": int(U_cnt.max())}
    return result(us_tok, "us/token", args.steps, args.warmup, total_ms / args.steps, config,
                  step_bytes=step_bytes,
                  step_GBps=round(step_bytes / (us_tok * 1e-6) / 1e9, 1),
                  step_frac_of_peak=round(step_bytes / (us_tok * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  step_stats=dist,
                  setup={"calibrate_ms": round(calib_ms, 2), "prefill_ms": round(prefill_ms, 2)},
                  roofline=roofline("rowop_wave_kernel<GLU> (gate/up over the compacted union)",
                                    glu_total / L, glu_us,
                                    measured_traffic("rowop_glu_selectinfer_decode",
                                                     ["rowop_b1.hip", "sffn_device.h"])),
                  fused_decode=fused,
                  cpu_baseline=cpu)


def fused_bytes(u: int, d: int) -> int:
    """One fused layer over u neurons: the gate, up and down bf16 rows of d
    per neuron, h read, the workgroups' fp32 partials written and read back
    by the reduction (G = min(256, ceil(u / 8)) of d each), h read and
    written by the reduction."""
    G = min(256, max(1, (u + 7) // 8))
    return 3 * u * d * 2 + 4 * d + 2 * G * d * 4 + 2 * 4 * d


def run_c1_fused(args, torch, stack, Xd, h, xcur, g_two, L, d, U_cnt, T):
    """The same decode with the fused per-neuron pass (one record of gate, up
    and down rows per neuron of U; a second launch adds the workgroup
    partials to the residual), timed the same way; plus the largest
    difference from the two-launch decode over one token."""
    stack.compact_records()

    def step():
        h.copy_(xcur)
        stack.decode_fused(h)

    gf = T.capture(step)
    for t in range(args.warmup):
        xcur.copy_(Xd[t])
        gf.replay()
    torch.cuda.synchronize()
    ms = T.replay_ms(gf, args.steps, before=lambda i: xcur.copy_(Xd[args.warmup + i]))
    us_tok = ms * 1e3 / args.steps
    xcur.copy_(Xd[0])
    g_two.replay()
    torch.cuda.synchronize()
    ref = h.clone()
    gf.replay()
    torch.cuda.synchronize()
    diff = float((h - ref).abs().max() / ref.pow(2).mean().sqrt())
    byts = int(sum(fused_bytes(int(u), d) for u in U_cnt))
    log(f"fused decode: {us_tok:.1f} us/token; max |fused - two-launch| / rms = {diff:.2e}")
    return {"kernels": "fused_swiglu_kernel + splitk_reduce_kernel per layer",
            "us_per_token": round(us_tok, 2), "us_per_layer": round(us_tok / L, 3),
            "bytes_per_token": byts, "GBps": round(byts / (us_tok * 1e-6) / 1e9, 1),
            "max_rel_diff_vs_two_launch": diff}


# ============================================================ c1-loading: SelectInfer Table 1 knobs

def run_c1_loading(args, torch, B, synth, P, T):
    cfg = synth.SHAPES["c1_loading"]
    L, N, d = cfg["layers"], cfg["n"], cfg["d"]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    layers = synth.ffn_stack(args.seed, synth.W_C1, L, N, d, threads=min(16, os.cpu_count() or 1))
    dev_layers = [tuple(P.to_device_bf16(m, dev) for m in lay) for lay in layers]
    log(f"weights: {L} layers x 3 x [{N} x {d}] bf16 in {time.perf_counter() - t0:.1f} s")
    pc = lambda k: P.pct_count(cfg[k], N)  # noqa: E731
    stack = P.SelectInferLoadedStack(dev_layers, pc("base_pct"), pc("loaded_pct"), pc("alpha_pct"),
                                     pc("computed_pct"), first=cfg["first"], last=cfg["last"],
                                     max_tokens=max(cfg["task_tokens"], cfg["prompt_tokens"],
                                                    3 * cfg["mixture_tokens_per_task"]))
    del dev_layers
    Xt = torch.from_numpy(synth.tokens(args.seed, synth.W_C1, 11, cfg["task_tokens"], d)).to(dev)
    Xm = torch.from_numpy(synth.mixture_tokens(args.seed, synth.W_C1, 12,
                                               cfg["mixture_tokens_per_task"], d)).to(dev)
    Xp = torch.from_numpy(synth.tokens(args.seed, synth.W_C1, 13, cfg["prompt_tokens"], d)).to(dev)
    n_tok = args.warmup + args.steps
    Xd_host = synth.tokens(args.seed, synth.W_C1, 14, n_tok, d)
    Xd = torch.from_numpy(Xd_host).to(dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    e0, e1, e2, e3 = ev(), ev(), ev(), ev()
    torch.cuda.synchronize()
    e0.record()
    stack.profile(Xt, Xm)
    e1.record()
    stack.load()
    e2.record()
    stack.release_full_weights()
    stack.prefill(Xp)          # includes the per-prompt compaction
    e3.record()
    torch.cuda.synchronize()
    profile_ms, load_ms, prefill_ms = e0.elapsed_time(e1), e1.elapsed_time(e2), e2.elapsed_time(e3)
    ks = [stack.comp[l][4] for l in range(L)]
    n_mod = len(stack.modified)
    resident = sum((stack.gamma_k if l in stack.modified else N) * 3 * d * 2 for l in range(L))
    log(f"profile {profile_ms:.1f} ms, load {load_ms:.1f} ms, prefill + compaction "
        f"{prefill_ms:.1f} ms; computed per layer {sorted(set(ks))}; resident FFN "
        f"{resident / 1e9:.2f} GB of {L * N * 3 * d * 2 / 1e9:.2f} GB")
    step_bytes = int(sum(glu_bytes(k, d) + down_bytes(k, d) for k in ks))
    glu_total = int(sum(glu_bytes(k, d) for k in ks))

    h = torch.zeros(d, dtype=torch.float32, device=dev)
    xcur = torch.zeros(d, dtype=torch.float32, device=dev)

    def step():
        h.copy_(xcur)
        stack.decode(h)

    g = T.capture(step)
    for t in range(args.warmup):
        xcur.copy_(Xd[t])
        g.replay()
    torch.cuda.synchronize()
    total_ms = T.replay_ms(g, args.steps, before=lambda i: xcur.copy_(Xd[args.warmup + i]))
    us_tok = total_ms * 1e3 / args.steps
    log(f"decode: {us_tok:.1f} us/token over {args.steps} steps")
    dist = T.step_stats(g, args.steps, before=lambda i: xcur.copy_(Xd[args.warmup + i]))
    gg = T.capture(lambda: [stack.decode_gate_up(l, h) for l in range(L)])
    glu_us = T.replay_ms(gg, args.steps) * 1e3 / (args.steps * L)
    log(f"gate/up (28 launches, mixed sizes): {glu_us:.2f} us/launch")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        U_pos, U_cnt = stack.U_pos.cpu().numpy(), stack.U_cnt.cpu().numpy()
        load_idx = stack.load_idx.cpu().numpy()
        ids = [load_idx[l][U_pos[l, :U_cnt[l]]] if l in stack.modified else np.arange(N)
               for l in range(L)]

        def one(i):
            hh = Xd_host[i % Xd_host.shape[0]].astype(np.float64)
            for l, (Wg, Wu, WdT) in enumerate(layers):
                _, y = oracle.decode_over_set(Wg, Wu, WdT, oracle.rms_normalize(hh, P.RMS_EPS),
                                              ids[l])
                hh = hh + y

        cpu = cpu_baseline(one, args.cpu_seconds,
                           "decode token(s) x 28 layers over the same computed sets, numpy fp64")

    config = {"workload": "SelectInfer 28-layer FFN stack, Llama3.2-3B shape, Table 1 knobs: layers "
                          "5..25 loaded selectively (base 30% by task-specific Eq (1) scores + "
                          "secondary by cross-task scores up to 70% resident) and computed over "
                          "40% (base + the most frequent of each prompt token's top 30% of loaded "
                          "neurons), layers 0-4 and 26-27 dense; decode at batch 1",
              "layers": L, "modified_layers": n_mod, "d_model": d, "d_ff": N, "batch": 1,
              "computed_per_modified_layer": stack.comp[min(stack.modified)][4],
              "resident_ffn_bytes": resident, "full_ffn_bytes": L * N * 3 * d * 2}
    return result(us_tok, "us/token", args.steps, args.warmup, total_ms / args.steps, config,
                  step_bytes=step_bytes,
                  step_GBps=round(step_bytes / (us_tok * 1e-6) / 1e9, 1),
                  step_frac_of_peak=round(step_bytes / (us_tok * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  step_stats=dist,
                  setup={"profile_ms": round(profile_ms, 2), "load_ms": round(load_ms, 2),
                         "prefill_ms": round(prefill_ms, 2)},
                  roofline=roofline("rowop_wave_kernel<GLU> (gate/up of every layer, mean launch)",
                                    glu_total / L, glu_us),
                  cpu_baseline=cpu)


# ============================================================ c0: per-token top-k layer

def run_c0(args, torch, B, synth, P, T):
    cfg = synth.SHAPES["c0"]
    N, d = cfg["n"], cfg["d"]
    keep = P.pct_count(cfg["keep_pct"], N)
    copies = 16      # 16 x 96 MiB of weights: far beyond the 256 MB Infinity Cache
    dev = torch.device("cuda:0")
    lay, host_w = [], None
    for c in range(copies):
        mats = [synth.weight_bf16(args.seed, synth.W_C0, c, 0, t, N, d)
                for t in (synth.T_GATE, synth.T_UP, synth.T_DOWN)]
        host_w = host_w or mats
        # the copies stand for successive layers: one set of intermediate
        # buffers (activations, index list, workspace) serves them all
        lay.append(P.SwigluSparseLayer(*[P.to_device_bf16(m, dev) for m in mats], keep,
                                       buffers_from=lay[0] if lay else None))
    n_tok = (args.steps + 2) * copies
    X_host = synth.tokens(args.seed, synth.W_C0, 0, n_tok, d)
    X = torch.from_numpy(X_host).to(dev)
    xbuf = torch.zeros(copies, d, dtype=torch.float32, device=dev)
    y = torch.zeros(copies, d, dtype=torch.float32, device=dev)

    def step():
        for c in range(copies):
            lay[c](xbuf[c], y[c])

    xbuf.copy_(X[0:copies])   # the capture's warm-up runs on real tokens
    gs = T.capture(step)
    total_ms = T.replay_ms(gs, args.steps,
                           before=lambda i: xbuf.copy_(X[i * copies:(i + 1) * copies]))
    us_tok = total_ms * 1e3 / (args.steps * copies)
    dist = T.step_stats(gs, args.steps, before=lambda i: xbuf.copy_(X[i * copies:(i + 1) * copies]),
                        per_step=copies)

    def glu_only():
        for c in range(copies):
            B.sparse_ffn_gemv(B.OP_GLU_SILU, lay[c].Wg, lay[c].Wu, xbuf[c], lay[c].a,
                              key_out=lay[c].key)

    # the layer's calls: the selection as a threshold, the keyed product
    def sel_only():
        for c in range(copies):
            B.sparse_ffn_select_threshold(lay[c].key, B.KEY_U32, keep, lay[c].thr)

    def down_only():
        for c in range(copies):
            B.sparse_ffn_gemv_keyed(lay[c].WdT, lay[c].a, lay[c].key, B.KEY_U32, lay[c].thr, keep,
                                    y[c], workspace=lay[c].ws)

    per = lambda body: T.replay_ms(T.capture(body), args.steps) * 1e3 / (args.steps * copies)  # noqa: E731
    glu_us, sel_us, down_us = per(glu_only), per(sel_only), per(down_only)
    glu_b = 2 * N * d * 2 + 4 * d + 8 * N
    sel_b = 4 * N + 8
    down_b = keyed_down_bytes(N, keep, d)
    step_b = glu_b + sel_b + down_b
    log(f"c0: {us_tok:.2f} us/token; gate/up {glu_us:.2f} us, select {sel_us:.2f} us, "
        f"gathered down {down_us:.2f} us")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        cpu = cpu_baseline(lambda i: oracle.sparse_swiglu_layer(*host_w, X_host[i], keep),
                           args.cpu_seconds, "token(s) through the layer, numpy fp64")
    config = {"workload": "single SwiGLU FFN layer, Llama3.2-1B shape (d_model 2048, d_ff 8192), "
                          "per-token top 50% by |silu(gate)*up|, batch 1 (16 rotating weight copies)",
              "d_model": d, "d_ff": N, "keep": keep, "batch": 1}
    return result(us_tok, "us/token", args.steps * copies, 2, total_ms / args.steps, config,
                  step_bytes=step_b, step_GBps=round(step_b / (us_tok * 1e-6) / 1e9, 1),
                  kernels_us={"gate_up_dense": round(glu_us, 3), "select": round(sel_us, 3),
                              "gathered_down": round(down_us, 3)},
                  roofline=roofline("axpy_keyed_kernel + splitk_reduce_kernel (gathered down "
                                    "over the kept 50%, rows formed from the keys, one call)",
                                    down_b, down_us,
                                    measured_traffic("axpy_b1_swiglu_top50_layer", AXPY_B1_SOURCES)),
                  dense_gate_up=roofline("rowop_wave_kernel<GLU> (dense gate/up, keys)", glu_b,
                                         glu_us,
                                         measured_traffic("rowop_glu_swiglu_top50_layer",
                                                          ["rowop_b1.hip", "sffn_device.h"])),
                  cpu_baseline=cpu,
                  step_stats=dist)


# ============================================================ c2: SpAx three-tier read

def run_c2(args, torch, B, synth, P, T):
    cfg = synth.SHAPES["c2"]
    d, dff = cfg["d"], cfg["d_ff"]
    n_qkv = sum(cfg["qkv_out"])
    seg_qkv = [0, cfg["qkv_out"][0], cfg["qkv_out"][0] + cfg["qkv_out"][1], n_qkv]
    copies = 8       # 8 x ~210 MB (bf16 + codes)
    dev = torch.device("cuda:0")
    kq_t, kq_m = P.pct_count(cfg["top_pct"], d), P.pct_count(cfg["mid_pct"], d)
    kd_t, kd_m = P.pct_count(cfg["top_pct"], dff), P.pct_count(cfg["mid_pct"], dff)
    projs = []
    for c in range(copies):
        Wq = synth.torch_weight_bf16(args.seed, synth.W_C2, c, 0, synth.T_QKV, d, n_qkv, dev)
        Wd = synth.torch_weight_bf16(args.seed, synth.W_C2, c, 0, synth.T_DOWN, dff, d, dev)
        wa = args.weight_aware
        # the copies stand for successive layers and share their tier lists
        # and workspaces
        projs.append((P.TieredProjection(Wq, seg_qkv, kq_t, kq_m, weight_aware=wa,
                                         buffers_from=projs[0][0] if projs else None),
                      P.TieredProjection(Wd, [0, d], kd_t, kd_m, weight_aware=wa,
                                         buffers_from=projs[0][1] if projs else None)))
    n_tok = copies * (args.steps + 2)
    Xq_host = synth.tokens(args.seed, synth.W_C2, 1, n_tok, d)
    Xd_host = synth.tokens(args.seed, synth.W_C2, 2, n_tok, dff)
    Xq, Xd = torch.from_numpy(Xq_host).to(dev), torch.from_numpy(Xd_host).to(dev)
    xq = torch.zeros(copies, d, dtype=torch.float32, device=dev)
    xd = torch.zeros(copies, dff, dtype=torch.float32, device=dev)
    yq = torch.zeros(copies, n_qkv, dtype=torch.float32, device=dev)
    yd = torch.zeros(copies, d, dtype=torch.float32, device=dev)

    def step():
        for c in range(copies):
            projs[c][0](xq[c], yq[c])
            projs[c][1](xd[c], yd[c])

    def before(i):
        xq.copy_(Xq[i * copies:(i + 1) * copies])
        xd.copy_(Xd[i * copies:(i + 1) * copies])

    before(0)   # the capture's warm-up runs on real tokens
    gs = T.capture(step)
    total_ms = T.replay_ms(gs, args.steps, before=before)
    us_tok = total_ms * 1e3 / (args.steps * copies)
    dist = T.step_stats(gs, args.steps, before=before, per_step=copies)

    keyed = projs[0][0].keyed

    def product(p, x, y):
        # the tiered product alone, on the tiers the last step selected
        if keyed:
            B.sparse_ffn_tiered_gemv_keyed(p.Wt, p.rec, p.seg_rows, x, x, B.KEY_ABS_F32, p.thr[0],
                                           p.thr[1], p.k_top, p.k_mid, y, workspace=p.ws)
        else:
            B.sparse_ffn_tiered_gemv(p.Wt, p.rec, p.seg_rows, x, p.idx_top, p.cnt[0:1], p.k_top,
                                     p.idx_mid, p.cnt[1:2], p.k_mid, y, workspace=p.ws)

    def down_only():
        for c in range(copies):
            product(projs[c][1], xd[c], yd[c])

    down_us = T.replay_ms(T.capture(down_only), args.steps) * 1e3 / (args.steps * copies)

    def qkv_only():
        for c in range(copies):
            product(projs[c][0], xq[c], yq[c])

    qkv_us = T.replay_ms(T.capture(qkv_only), args.steps) * 1e3 / (args.steps * copies)
    rec_q, rec_d = projs[0][0].rec.shape[1], projs[0][1].rec.shape[1]
    if keyed:
        # selected bf16 rows and records, x once (it is also the key), the two pairs, y
        qkv_b = kq_t * n_qkv * 2 + kq_m * rec_q + 4 * d + 16 + 4 * n_qkv
        down_b = kd_t * d * 2 + kd_m * rec_d + 4 * dff + 16 + 4 * d
        step_b = qkv_b + down_b + (4 * d + 4 * dff)    # the selections read x
    else:
        qkv_b = kq_t * n_qkv * 2 + kq_m * rec_q + 8 * (kq_t + kq_m) + 4 * n_qkv
        down_b = kd_t * d * 2 + kd_m * rec_d + 8 * (kd_t + kd_m) + 4 * d
        # selection reads x (and the column norms when weight-aware), the product x again
        step_b = qkv_b + down_b + (3 if args.weight_aware else 2) * (4 * d + 4 * dff)
    log(f"c2: {us_tok:.2f} us/token; tiered down {down_us:.2f} us, tiered QKV {qkv_us:.2f} us")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        Wq0 = projs[0][0].Wt.cpu().numpy().view(np.uint16)
        Wd0 = projs[0][1].Wt.cpu().numpy().view(np.uint16)
        encq, encd = oracle.encode_4bit(Wq0, seg_qkv), oracle.encode_4bit(Wd0, [0, d])
        if args.weight_aware:
            nq = oracle.row_norms(Wq0).astype(np.float32)
            nd = oracle.row_norms(Wd0).astype(np.float32)
            sets = lambda x, kt, km, nrm: oracle.weighted_tier_sets(x, nrm, kt, km)  # noqa: E731
        else:
            nq = nd = None
            sets = lambda x, kt, km, nrm: oracle.tier_sets(x, kt, km)  # noqa: E731

        def one(i):
            tq, mq = sets(Xq_host[i], kq_t, kq_m, nq)
            oracle.tiered_gemv(Wq0, *encq, seg_qkv, Xq_host[i], tq, mq)
            td, md = sets(Xd_host[i], kd_t, kd_m, nd)
            oracle.tiered_gemv(Wd0, *encd, [0, d], Xd_host[i], td, md)

        cpu = cpu_baseline(one, args.cpu_seconds,
                           "token(s) (QKV + down tiers and products; encoding excluded), "
                           "numpy fp64")
    config = {"workload": "SpAx three-tier read, Llama3.1-8B shape: QKV 4096->4096/1024/1024 and "
                          "down 14336->4096; 15% bf16 / 35% 4-bit / 50% skipped by "
                          + ("|x_j| * ||W[:, j]||_2 (WiSparse weight-aware)" if args.weight_aware
                             else "|x|")
                          + "; batch 1 (8 rotating weight copies)"
                          + ("; tiers as threshold pairs read by the product" if keyed else ""),
              "batch": 1, "tiers_qkv": [kq_t, kq_m], "tiers_down": [kd_t, kd_m]}
    return result(us_tok, "us/token", args.steps * copies, 2, total_ms / args.steps, config,
                  step_bytes=step_b, step_GBps=round(step_b / (us_tok * 1e-6) / 1e9, 1),
                  dense_equivalent_bytes=(d * n_qkv + dff * d) * 2,
                  roofline=roofline("tiered_kernel (down 14336->4096, 15% bf16 + 35% 4-bit)",
                                    down_b, down_us,
                                    None if args.weight_aware else
                                    measured_traffic("tiered_down_spax",
                                                     ["tiered.hip", "axpy_b1.hip", "sffn_device.h"])),
                  cpu_baseline=cpu,
                  step_stats=dist)


# ============================================================ c3: ReLU-sparse MoE stack

def run_c3(args, torch, B, synth, P, T):
    cfg = synth.SHAPES["c3"]
    L, E, N, d, S = cfg["layers"], cfg["experts"], cfg["n"], cfg["d"], cfg["cluster"]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    experts = [[(synth.torch_weight_bf16(args.seed, synth.W_C3, l, e, synth.T_GATE, N, d, dev,
                                         cluster=S),
                 synth.torch_weight_bf16(args.seed, synth.W_C3, l, e, synth.T_UP, N, d, dev),
                 synth.torch_weight_bf16(args.seed, synth.W_C3, l, e, synth.T_DOWN, N, d, dev))
                for e in range(E)] for l in range(L)]
    torch.cuda.synchronize()
    log(f"c3 weights: {L} x {E} x 3 x [{N} x {d}] bf16 on the device in "
        f"{time.perf_counter() - t0:.1f} s")
    steps = min(args.steps, cfg["decode_tokens"])
    logits = torch.from_numpy(synth.router_logits(args.seed, synth.W_C3, L, steps, E)).to(dev)
    X_host = synth.tokens(args.seed, synth.W_C3, 1, steps, d)
    X = torch.from_numpy(X_host).to(dev)
    tau_scale = cfg["zero_frac_quantile"] * synth.WEIGHT_STD
    nc = N // S
    if args.predictor:
        bias = torch.from_numpy(synth.predictor_bias(nc, d, cfg["pred_theta"], cfg["pred_frac"])).to(dev)
        preds = [[(synth.torch_weight_bf16(args.seed, synth.W_C3, l, e, synth.T_PRED, nc, d, dev),
                   bias) for e in range(E)] for l in range(L)]
        moe = P.PredictedMoEStack(experts, preds, S, tau_scale=tau_scale, theta=cfg["pred_theta"])
    else:
        moe = P.ReluMoEStack(experts, S, tau_scale=tau_scale)
    moe.route(logits)
    h = torch.zeros(d, dtype=torch.float32, device=dev)

    # An untimed eager pass records the active-cluster counts (exact bytes
    # read); then one graph per token (the routed experts differ per token).
    counts = np.zeros((steps, L, 2), dtype=np.int64)
    saved = []     # token 0, per layer: routed experts and their cluster lists
    for t in range(steps):
        h.copy_(X[t])

        def rec(l, tt, hh, chosen, t=t):
            ci, cc = (moe.pidx[l & 1], moe.pcnt[l & 1]) if args.predictor else (moe.cidx, moe.ccnt)
            counts[t, l] = cc.cpu().numpy()
            if t == 0:
                saved.append((list(chosen), ci.clone(), cc.clone()))
        moe.decode(h, t, record=rec)
    graphs = [T.capture(lambda t=t: (h.copy_(X[t]), moe.decode(h, t))) for t in range(steps)]
    for g in graphs[:2]:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for g in graphs:
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    us_tok = total_ms * 1e3 / steps
    dist = T.step_stats(graphs, steps)
    if args.predictor:
        # per routed expert: predictor rows, bias, logits and keys; per
        # predicted cluster: gate, up and down rows, a written and read
        gate_b = nc * d * 2 + 4 * d + 3 * 4 * nc
        clus_b = 3 * S * d * 2 + 2 * 4 * S
    else:
        gate_b = N * d * 2 + 4 * d + 4 * N
        clus_b = 2 * S * d * 2 + 3 * 4 * S      # up + down rows, r read, a written and read
    step_b = int(L * 2 * (gate_b + 4 * nc) + counts.sum(axis=(1, 2)).mean() * clus_b)
    log(f"c3: {us_tok:.1f} us/token, {step_b / 1e9:.2f} GB/token, "
        f"{'predicted' if args.predictor else 'active'} clusters {counts.mean() / nc:.3f}")

    if args.predictor:
        # dominant kernel: the ReGLU over each routed expert's predicted clusters
        def dom():
            for l in range(L):
                for j, e in enumerate(moe.route_host[l * moe.T]):
                    Wg, Wu, _ = experts[l][e]
                    B.sparse_ffn_gemv(B.OP_GLU_RELU, Wg, Wu, h, moe.a[j], idx=moe.pidx[0, j],
                                      count=moe.pcnt[0, j:j + 1], k_max=nc, group=S,
                                      tau_scale=moe.tau_scale, rms_eps=moe.rms_eps)
        moe.predict(0, 0, h)
        torch.cuda.synchronize()
        dom_count = int(moe.pcnt[0].sum().item())
        dom_b = dom_count * S * (2 * d * 2 + 4) / 2 + 4 * d
        dom_name = "rowop_wave_kernel<GLU_RELU> (gate + up over predicted clusters)"
    else:
        def dom():
            for l in range(L):
                for j, e in enumerate(moe.route_host[l * moe.T]):
                    B.sparse_ffn_gemv(B.OP_DOT_RELU, experts[l][e][0], None, h, moe.r[j],
                                      tau_scale=moe.tau_scale, rms_eps=moe.rms_eps)
        dom_b = gate_b
        dom_name = "rowop_wave_kernel<DOT_RELU> (dense expert gate)"

    gate_us = T.replay_ms(T.capture(dom), 16) * 1e3 / (16 * L * 2)

    # The gathered part of each layer, replayed alone over token 0's cluster
    # lists: the routed experts' ups (or fused ReGLUs) over their clusters in
    # one launch, then both down products in one gathered product.
    hs = torch.zeros(d, dtype=torch.float32, device=dev)

    def gathered():
        for l, (chosen, ci, cc) in enumerate(saved):
            k = len(chosen)
            ex = [experts[l][e] for e in chosen]
            idx, cnt = [ci[j] for j in range(k)], [cc[j:j + 1] for j in range(k)]
            a = [moe.a[j] for j in range(k)]
            if args.predictor:
                B.sparse_ffn_rowop_lists(B.OP_GLU_RELU, [m[0] for m in ex], [m[1] for m in ex], h,
                                         a, idxs=idx, counts=cnt, k_maxs=[nc] * k, group=S,
                                         tau_scale=moe.tau_scale, rms_eps=moe.rms_eps)
            else:
                B.sparse_ffn_rowop_lists(B.OP_GATED, None, [m[1] for m in ex], h, a, idxs=idx,
                                         counts=cnt, k_maxs=[nc] * k, group=S,
                                         auxs=[moe.r[j] for j in range(k)], rms_eps=moe.rms_eps)
            B.sparse_ffn_gemv_lists([m[2] for m in ex], a, idx, cnt, [nc] * k, hs, group=S,
                                    alphas=[moe.route_w[l * moe.T, j:j + 1] for j in range(k)],
                                    accumulate=True, workspace=moe.ws)

    gath_us = T.replay_ms(T.capture(gathered), max(4, steps)) * 1e3 / (max(4, steps) * L)
    c0 = counts[0].sum(axis=1)      # clusters of both routed experts, per layer, token 0
    rows_per_cluster_b = S * d * 2 * (3 if args.predictor else 2)   # (gate,) up, down rows
    gath_b = float(np.mean(c0 * (rows_per_cluster_b + S * 12 + 8) + 12 * d))

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        l_s = [0, L // 2, L - 1]
        host = {(l, e): tuple(m.cpu().numpy().view(np.uint16) for m in experts[l][e])
                for l in l_s for e in moe.route_host[l * moe.T]}
        if args.predictor:
            pred_host = {(l, e): preds[l][e][0].cpu().numpy().view(np.uint16)
                         for l in l_s for e in moe.route_host[l * moe.T]}
            bias_h = bias.cpu().numpy()
            theta32 = float(np.float32(cfg["pred_theta"]))

        def one(i):
            l = l_s[i % len(l_s)]
            x = oracle.rms_normalize(X_host[0], P.RMS_EPS)
            tau = oracle.relu_threshold(x, cfg["zero_frac_quantile"], synth.WEIGHT_STD)
            for j, e in enumerate(moe.route_host[l * moe.T]):
                if args.predictor:
                    Wp = pred_host[(l, e)]
                    cl = oracle.predicted_clusters(oracle.predictor_logits(Wp, bias_h, x), theta32)
                    oracle.predicted_expert(*host[(l, e)], x, tau, cl, S)
                else:
                    oracle.relu_expert(*host[(l, e)], x, tau, S)

        cpu = cpu_baseline(one, args.cpu_seconds,
                           f"layer(s) of 2 routed experts "
                           f"({'predictor, ' if args.predictor else 'gate, '}clusters, up, down) "
                           f"at token 0, numpy fp64, scaled to {L} layers", scale=L * 1e6)
    config = {"workload": "ReLU-sparse MoE FFN stack, TurboSparse-Mixtral-like: 32 layers x 8 "
                          "experts (d_model 4096, d_ff 14336), top-2 router, ~90% exact zeros, "
                          "32-row clusters, batch 1"
                          + ("; clusters from a random online predictor per layer and expert "
                             "(sigmoid(W_pred h + b) > 0.45 on the previous layer's input, "
                             "~20% of clusters), no dense gate" if args.predictor else ""),
              "layers": L, "experts": E, "batch": 1,
              ("predicted_cluster_frac" if args.predictor else "active_cluster_frac"):
                  round(float(counts.mean() / nc), 4)}
    gname = ("rowop_lists_kernel<GLU_RELU> + axpy_lists_kernel + splitk_reduce_kernel (gate, up "
             "and down rows of the predicted clusters of both routed experts, one layer)"
             if args.predictor else
             "rowop_lists_kernel<GATED> + axpy_lists_kernel + splitk_reduce_kernel (up and down "
             "rows of the active clusters of both routed experts, one layer)")
    log(f"c3 gathered part: {gath_us:.2f} us/layer for {gath_b / 1e6:.1f} MB")
    return result(us_tok, "us/token", steps, 2, total_ms / steps, config, step_bytes=step_b,
                  step_GBps=round(step_b / (us_tok * 1e-6) / 1e9, 1),
                  kernels_us={"dense_part_per_expert": round(gate_us, 3),
                              "gathered_part_per_layer": round(gath_us, 3)},
                  roofline=roofline(gname, gath_b, gath_us,
                                    measured_traffic("moe_gathered_layer_predictor" if args.predictor
                                                     else "moe_gathered_layer",
                                                     ["rowop_b1.hip"] + AXPY_B1_SOURCES)),
                  dense_part=roofline(dom_name, dom_b, gate_us,
                                      None if args.predictor else
                                      measured_traffic("rowop_relu_gate_moe",
                                                       ["rowop_b1.hip", "sffn_device.h"])),
                  cpu_baseline=cpu,
                  step_stats=dist)


# ============================================================ c4: batched union on MFMA

def run_c4(args, torch, B, synth, P, T):
    cfg = synth.SHAPES["c4"]
    N, d, batch = cfg["n"], cfg["d"], args.batch
    keep = P.pct_count(cfg["keep_pct"], N)
    copies = 4       # 4 x ~535 MB
    dev = torch.device("cuda:0")
    lays = []
    for c in range(copies):
        w = [synth.torch_weight_bf16(args.seed, synth.W_C4, c, 0, t, N, d, dev)
             for t in (synth.T_GATE, synth.T_UP, synth.T_DOWN)]
        # the copies stand for successive layers and share their buffers
        lays.append(P.BatchedUnionLayer(*w, keep, batch, buffers_from=lays[0] if lays else None,
                                        packed=args.layout == "packed",
                                        union_list=args.union == "list"))
    n_b = args.steps + 2
    X_host = synth.tokens(args.seed, synth.W_C4, batch, n_b * copies * batch, d)
    X = torch.from_numpy(X_host).to(dev).view(n_b * copies, batch, d)
    xb = torch.zeros(copies, batch, d, dtype=torch.float32, device=dev)
    Y = torch.zeros(copies, batch, d, dtype=torch.float32, device=dev)

    def step():
        for c in range(copies):
            lays[c](xb[c], Y[c])

    xb.copy_(X[0:copies])   # the capture's warm-up runs on real tokens (zeros would tie every key)
    gs = T.capture(step)
    total_ms = T.replay_ms(gs, args.steps,
                           before=lambda i: xb.copy_(X[i * copies:(i + 1) * copies]))
    us_batch = total_ms * 1e3 / (args.steps * copies)
    dist = T.step_stats(gs, args.steps, before=lambda i: xb.copy_(X[i * copies:(i + 1) * copies]),
                        per_step=copies * batch)
    if lays[0].keyed:   # batch 1: the token's set, from its threshold pair
        u = float(np.mean([P.threshold_members(l.K.cpu().numpy(), l.thr.cpu().numpy()).size
                           for l in lays]))
    else:               # union sizes from the token masks
        u = float(np.mean([int((l.M != 0).any(dim=0).sum()) for l in lays]))
    masked = batch > 1 and not lays[0].union_list

    def weights(l):
        return (l.Pg, l.Pu, l.Pd) if l.packed else (l.Wg, l.Wu, l.WdT)

    def glu_only():
        for c in range(copies):
            Wg, Wu, _ = weights(lays[c])
            B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wu, xb[c], lays[c].A,
                              key_out=lays[c].K, workspace=lays[c].ws)

    def down_only():
        for c in range(copies):
            l = lays[c]
            if masked:   # the union formed in the product from the token masks
                B.sparse_ffn_gemv(B.OP_AXPY | B.MASKED_ROWS, weights(l)[2], None, l.A, Y[c],
                                  row_mask=l.M, workspace=l.ws)
                continue
            if l.keyed:  # batch 1: the rows the token's threshold selects (as the layer)
                B.sparse_ffn_gemv_keyed(weights(l)[2], l.A, l.K, B.KEY_U32, l.thr, keep, Y[c],
                                        workspace=l.ws)
                continue
            # the listed union (union_list)
            B.sparse_ffn_gemv(B.OP_AXPY, weights(l)[2], None, l.A, Y[c], idx=l.U, count=l.cnt,
                              k_max=N, row_mask=l.M if batch > 1 else None, workspace=l.ws)

    per = lambda body: T.replay_ms(T.capture(body), args.steps) * 1e3 / (args.steps * copies)  # noqa: E731
    glu_us, down_us = per(glu_only), per(down_only)
    glu_b = 2 * N * d * 2 + batch * (4 * d + 8 * N)
    if masked:   # union rows, every token's mask (the union is formed from them), activations
        down_b = int(u * d * 2 + batch * (N + 4 * u + 4 * d))
    elif lays[0].keyed:   # the token's rows, every key, its activations, the threshold, outputs
        down_b = keyed_down_bytes(N, int(round(u)), d)
    else:        # union rows and their indices, per token activations (+ masks), outputs
        down_b = int(u * d * 2 + 4 * u + batch * ((5 if batch > 1 else 4) * u + 4 * d))
    step_b = int(glu_b + down_b + batch * 5 * N)
    # at batch 1 the same calls run the wave-per-row kernel and the split-K gathered product
    k_glu, k_down = (("gate_up_mfma", "union_down_mfma") if batch > 1
                     else ("gate_up_rows", "union_down_keyed"))
    log(f"c4 batch {batch}: {us_batch:.2f} us/batch, union {u:.0f}; {k_glu} {glu_us:.2f} us, "
        f"{k_down} {down_us:.2f} us")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        w0 = [m.cpu().numpy().view(np.uint16) for m in (lays[0].Wg, lays[0].Wu, lays[0].WdT)]
        cpu = cpu_baseline(lambda i: oracle.batched_union_decode(
            *w0, X_host[i * batch:(i + 1) * batch], keep), args.cpu_seconds,
            f"batch(es) of {batch} tokens, numpy fp64", per_unit=batch)
    config = {"workload": f"batched decode, Qwen-27B-like layer (d_model 5120, d_ff 17408), "
                          f"per-token top 40%, union gathered once and contracted on MFMA, "
                          f"batch {batch} (4 rotating weight copies)",
              "d_model": d, "d_ff": N, "batch": batch, "union_mean": u,
              "weight_layout": ("packed: gate/up in 16-row x 128 tiles, down in 256-column panels"
                                if lays[0].packed else "row-major"),
              "union": ("formed in the product from the token masks" if masked
                        else "the token's own set, a threshold read by the keyed product"
                        if lays[0].keyed
                        else "listed by frequency counts and a union select")}
    return result(us_batch / batch, "us/token", args.steps * copies, 2, total_ms / args.steps,
                  config, us_per_batch=round(us_batch, 3), step_bytes=step_b,
                  step_GBps=round(step_b / (us_batch * 1e-6) / 1e9, 1),
                  kernels_us={k_glu: round(glu_us, 3), k_down: round(down_us, 3)},
                  roofline=roofline(("axpy_mfma_kernel + splitk_reduce_kernel (the union's down "
                                     "rows read once, per-token masks, one call)" if batch > 1
                                     else "axpy_keyed_kernel + splitk_reduce_kernel (the token's "
                                     "down rows, formed from its keys, one call)"),
                                    down_b, down_us,
                                    measured_traffic(f"union_down_b{batch}",
                                                     AXPY_MFMA_SOURCES if batch > 1
                                                     else AXPY_B1_SOURCES)),
                  dense_gate_up=roofline("rowop_mfma_kernel<GLU> (batched gate/up)" if batch > 1
                                         else "rowop_wave_kernel<GLU> (gate/up, batch 1)", glu_b,
                                         glu_us),
                  cpu_baseline=cpu,
                  step_stats=dist)


# ============================================================ all: the headline stack and every workload

SUB_KEYS_DROPPED = ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "dtype",
                    "weight_dtype", "data")


def run_all(args, torch, B, synth, P, T):
    """The SelectInfer stack as the line's value, then every other workload
    under "configs" (each with its gathered kernel as the roofline and a
    shorter CPU-oracle sample)."""
    import gc

    out = run_c1(args, torch, B, synth, P, T)
    subs = [("c0", dict(workload="c0")), ("c2", dict(workload="c2")), ("c3", dict(workload="c3"))]
    subs += [(f"c4_b{b}", dict(workload="c4", batch=b)) for b in (1, 4, 8, 16)]
    fns = {"c0": run_c0, "c2": run_c2, "c3": run_c3, "c4": run_c4}
    configs = {}
    for name, over in subs:
        gc.collect()
        torch.cuda.empty_cache()
        a = argparse.Namespace(**vars(args))
        a.cpu_seconds = args.cpu_seconds_sub
        a.predictor = a.weight_aware = False
        for k, v in over.items():
            setattr(a, k, v)
        t0 = time.perf_counter()
        r = fns[a.workload](a, torch, B, synth, P, T)
        configs[name] = {k: v for k, v in r.items() if k not in SUB_KEYS_DROPPED}
        rf = r["roofline"]
        log(f"{name}: {r['value']:.2f} {r['unit']}; gathered kernel {rf['launch_us']:.2f} us "
            f"= {rf['achieved']:.0f} GB/s ({100 * rf['frac']:.1f}% of peak) "
            f"[{time.perf_counter() - t0:.0f} s]")
    out["configs"] = configs
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    from activation_sparse_decode_amd import binding as B
    from activation_sparse_decode_amd import pipelines as P
    from activation_sparse_decode_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.lib()
    T = Timer(torch)
    run = {"all": run_all, "c0": run_c0, "c1": run_c1, "c1-loading": run_c1_loading, "c2": run_c2,
           "c3": run_c3, "c4": run_c4}[args.workload]
    out = run(args, torch, B, synth, P, T)
    props = torch.cuda.get_device_properties(0)
    out["env"] = {"device": props.name, "arch": getattr(props, "gcnArchName", None),
                  "compute_units": props.multi_processor_count,
                  "hip": torch.version.hip, "torch": torch.__version__, **clock_info(torch)}

    # A plain device copy of known size: the reference that scales the HBM
    # counters (FETCH_SIZE / WRITE_SIZE) of profiled kernels to bytes.
    calib = torch.empty(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    torch.empty_like(calib).copy_(calib)
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def clock_info(torch=None) -> dict:
    """The GPU's current core and memory clock levels (the amdgpu sysfs
    files of device 0's PCI function, the entry marked current) and the
    driver version, best effort: a missing file only drops its field.  Plain
    file reads: no tool is started, so a profiler's preload in this process
    is never carried into another program."""
    info = {}
    try:
        prop = torch.cuda.get_device_properties(0)
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (prop.pci_domain_id, prop.pci_bus_id,
                                                         prop.pci_device_id)
        clocks = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            with open(f"{dev}/{name}") as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            if cur:
                clocks[name[-4:]] = cur[0].rstrip("* ").split(":", 1)[-1].strip()
        if clocks:
            info["clocks"] = clocks
    except Exception:   # noqa: BLE001 -- absent files or properties only drop the field
        pass
    try:
        with open("/sys/module/amdgpu/version") as f:
            info["amdgpu_driver"] = f.read().strip()
    except OSError:
        pass
    return info


if __name__ == "__main__":
    main()
