"""Batch-1 decode throughput of the fused layer stack on one MI355X.

A step is one decode token through the whole stack: the embedding gather,
every layer's five fused kernels (RMSNorm+QKV+RoPE+append, split-K
attention, O projection + residual, RMSNorm+gate/up+SwiGLU, down projection
+ residual), and the position advance, replayed from one HIP graph. Inputs
(weights, synthetic cache prefill, tokens) are seeded, synthetic and resident
in HBM before timing starts.

Reported (one JSON line): tok/s of the stack, the achieved HBM bandwidth of
the token ((weight + KV bytes) per token x tok/s), a roofline entry for the
dominant kernel (the gated FFN) timed per launch with HIP events on its
launch stream, and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4]
                       [--unfused] [--eager] [--null-kernels] [--no-cpu]
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
PROFILES = os.path.join(ROOT, "profiles")
# sources whose code the gated-FFN kernel is built from
FFN_SOURCES = ["transformer_layer_amd/csrc/dec_gemv.h", "transformer_layer_amd/csrc/dec_device.h",
               "transformer_layer_amd/csrc/dec_internal.h", "transformer_layer_amd/csrc/dec_gemv_dense.hip",
               "transformer_layer_amd/csrc/dec_gemv_q4.hip", "transformer_layer_amd/csrc/dec_q4mfma.h"]


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def build_stack(cfg, flags, chunk):
    import torch
    import synth
    from transformer_layer_amd.engine import DecodeStack

    st = DecodeStack(cfg, flags=flags, attn_chunk=chunk)
    t0 = time.time()
    for l in range(cfg.n_layers):
        st.set_layer(l, synth.layer_weights(cfg, l))
        if cfg.ctx and not cfg.real_prefill:
            st.set_prefill(l, *synth.prefill(cfg, l))
        if l % 8 == 7:
            log(f"uploaded {l + 1}/{cfg.n_layers} layers ({time.time() - t0:.0f}s)")
    st.set_embedding(synth.embedding(cfg))
    torch.cuda.synchronize()
    return st


def ffn_kernel_time(st, cfg, reps: int):
    """Average duration of one gated-FFN launch, from HIP events on the
    stream the kernels run on. The kernel is launched for every layer of the
    stack back to back (each layer's own weights, so nothing stays cached);
    that sweep is captured once into a HIP graph, as the decode step launches
    its kernels, and replayed `reps` times between one pair of events, so the
    average includes the steady-state boundary between consecutive launches.
    Returns (graph-replayed seconds per launch, launches timed, host-launched
    seconds per launch): the same sweep launched from the host one kernel at a
    time, for comparison (it also pays each launch's host-side submission)."""
    import torch
    from transformer_layer_amd import lib as L

    n = reps * cfg.n_layers

    def sweep(sp):
        for l in range(cfg.n_layers):
            w, s = st.wstruct[l], st.state[l]
            L.dec_gated_ffn(st.desc, w.ffn_norm, w.wgate, w.wup, s.x, s.h, sp)

    def timed(run):
        stream = torch.cuda.current_stream()
        run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    t_host = timed(lambda: sweep(torch.cuda.current_stream().cuda_stream))
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sweep(torch.cuda.current_stream().cuda_stream)
    t_graph = timed(g.replay)
    return t_graph, n, t_host


def ffn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per gated-FFN launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when
    there is none for this workload or the kernel sources changed since."""
    path = os.path.join(PROFILES, f"gated_ffn_{cfg.name}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != ffn_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calib_copy(mb: int) -> None:
    """A plain streaming kernel of known size (dst = src + 1: reads and
    writes `mb` MiB), for scaling the byte counters. An elementwise kernel,
    not a DMA copy, so the counters see it."""
    import torch
    n = (mb << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"calibration kernel: {mb} MiB read + {mb} MiB written, 3 times")


def head_timing(st, cfg, lo: int, hi: int, steps: int, warmup: int) -> dict:
    """The token with the LM head: final RMSNorm, head GEMV and greedy argmax
    into the device token, which the next token's embedding reads (no
    teacher forcing), replayed from one graph. Also the head alone (GEMV +
    argmax, two kernels) timed back to back with HIP events on its stream.
    The head's bytes (vocab x hidden weights + norm) are not part of the
    stack's bytes per token."""
    import torch
    import synth

    glob_w = synth.model_globals(cfg)
    st.set_head(glob_w["final_norm"], glob_w["head"])
    toks = synth.tokens(cfg, 1)
    st.set_pos(lo)
    st.set_token(int(toks[0]))
    g = st.capture(lo, hi, greedy=True)
    st.set_pos(lo)
    st.set_token(int(toks[0]))
    for _ in range(warmup):
        g.replay()
    st.set_pos(lo)
    st.set_token(int(toks[0]))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    reps = 50
    st.head_step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        st.head_step()
    e1.record(stream)
    torch.cuda.synchronize()
    head_us = e0.elapsed_time(e1) * 1e3 / reps
    hb = synth.head_bytes(cfg)
    log(f"with head: {1e3 / ms:.1f} tok/s, {ms:.3f} ms/token; head alone {head_us:.1f} us "
        f"({hb / head_us / 1e3:.0f} GB/s)")
    return {"tok_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4), "head_us": round(head_us, 2),
            "head_bytes": int(hb), "head_gbs": round(hb / head_us / 1e3, 1), "vocab": cfg.vocab,
            "head_weights": glob_w["head"].kind, "kernels": 2}


def cpu_baseline(cfg, budget_s: float = 15.0):
    """The oracle (NumPy, float64) on a bounded sample: the first layers of
    the same stack for one decode token at the first decode position, scaled
    to tok/s of the whole stack."""
    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    per_layer = []
    n = 0
    tok = int(synth.tokens(cfg)[0])
    x = synth.embedding(cfg).data[tok].astype(np.float64)
    t_all = time.time()
    while n < cfg.n_layers:
        o = oracle.Oracle(cfg, [synth.layer_weights(cfg, n)])
        if cfg.ctx and not cfg.real_prefill:
            o.load_prefill(0, *synth.prefill(cfg, n))
        t0 = time.perf_counter()
        x = o.layer(0, x, cfg.ctx)
        per_layer.append(time.perf_counter() - t0)
        n += 1
        if sum(per_layer) >= budget_s or time.time() - t_all > 4 * budget_s:
            break
    t_layer = float(np.mean(per_layer))
    tok_s = 1.0 / (t_layer * cfg.n_layers)
    return {"value": tok_s, "unit": "tok/s", "cores": int(min(cores, blas_threads)) if blas_threads else cores,
            "kind": "oracle",
            "sample": f"layers 0..{n - 1} of the {cfg.n_layers}-layer stack, one decode token at position "
                      f"{cfg.ctx} (float64 NumPy, weights decoded from their storage type at use); "
                      f"{t_layer * 1e3:.0f} ms/layer scaled to the whole stack",
            "host_cores_available": cores, "blas_threads": blas_threads}


def timed_token_bytes(cfg, steps: int) -> float:
    """Algorithmic bytes per token over the positions a timed run of `steps`
    graph replays visits: ctx, ctx + 1, ..., wrapping to ctx after the
    decode window as the position advance does. Weights and norms of every
    layer, the KV read over 0..p and the KV write (synth.token_bytes's
    terms), the read averaged over the positions actually timed."""
    import synth
    mean_len = sum(cfg.ctx + (i % cfg.steps) + 1 for i in range(steps)) / steps
    kv = synth.kv_bytes(cfg, 1)
    wb = sum(synth.layer_weight_bytes(cfg).values())
    return cfg.n_layers * (wb + kv["read"] * mean_len + kv["write"])


def gpu_clocks() -> dict:
    """Current GPU clocks as rocm-smi reports them (best effort)."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=15).stdout
    except Exception as e:  # pragma: no cover
        return {"error": str(e)}
    clk = {}
    for line in out.splitlines():
        low = line.lower()
        for key in ("sclk", "mclk", "fclk", "socclk"):
            if f"{key} clock level" in low and "(" in line:
                clk[key] = line.split("(")[-1].split(")")[0]
    return clk or {"raw": out[-400:]}


class Workload:
    """One stack on the GPU with its per-token graph, ready to time."""

    def __init__(self, cfg, flags=0, chunk=0, eager=False):
        import synth
        self.cfg = cfg
        self.st = build_stack(cfg, flags, chunk)
        self.toks = synth.tokens(cfg, cfg.steps)
        self.st.set_token_list(self.toks)
        self.lo, self.hi = cfg.ctx, cfg.ctx + cfg.steps
        self.reset()
        if eager:
            self.step = lambda: self.st.token_step(self.lo, self.hi)  # noqa: E731
        else:
            self.graph = self.st.capture(self.lo, self.hi)
            self.reset()
            self.step = self.graph.replay

    def reset(self):
        self.st.set_pos(self.lo)
        self.st.set_token(int(self.toks[0]))

    def timed(self, steps: int, warmup: int):
        """Warm up, reset the position, then time exactly `steps` tokens with
        HIP events on the current stream. Returns (ms, wall seconds)."""
        import torch
        for _ in range(warmup):
            self.step()
        self.reset()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            self.step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), time.perf_counter() - t_wall

    def close(self):
        import torch
        self.graph = None
        self.step = None
        self.st = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def workload_config(spec: str):
    """A workload by name, optionally over another KV cache type or cached
    length: "C5", "C5:i8" (the same stack over an int8 cache), "C5@32768"
    (32768 cached positions), "C5:i8@32768"."""
    import synth
    spec, _, ctx = spec.partition("@")
    name, _, kv = spec.partition(":")
    cfg = synth.CONFIGS[name]
    if kv and kv != cfg.kvtype:
        cfg = cfg.with_(kvtype=kv, name=f"{cfg.name}_{kv}kv")
    if ctx and int(ctx) != cfg.ctx:
        cfg = cfg.with_(ctx=int(ctx), name=f"{cfg.name}_ctx{int(ctx)}")
    return cfg


def other_workload(spec: str, steps: int, warmup: int, repeats: int) -> dict:
    """tok/s of another workload's stack: the median of `repeats` timed runs
    of `steps` tokens (same protocol as the headline)."""
    cfg = workload_config(spec)
    name = spec.partition("@")[0].partition(":")[0]
    log(f"config {cfg.name}: building stack ({cfg.n_layers} layers)")
    w = Workload(cfg)
    runs = []
    for r in range(repeats):
        ms, _ = w.timed(steps, warmup if r == 0 else 2)
        runs.append(steps / (ms * 1e-3))
    err = w.st.check_err()
    w.close()
    tok_s = float(np.median(runs))
    bpt = timed_token_bytes(cfg, steps)
    gbs = bpt * tok_s / 1e9
    out = {"tok_s": round(tok_s, 2), "tok_s_runs": [round(v, 2) for v in runs], "ms_per_step": round(1e3 / tok_s, 4),
           "bytes_per_token": int(bpt), "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "layers": cfg.n_layers, "weights": cfg.wtype, "kv_cache": cfg.kvtype, "context": cfg.ctx,
           "device_error": err}
    if name in ("C3", "C4", "C5"):
        out["target_70pct_tok_s"] = round(0.7 * PEAK_HBM_GBS * 1e9 / bpt, 1)
    log(f"{cfg.name}: {tok_s:.1f} tok/s, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.3f} of peak)")
    return out


def ab_modes(cfg, steps: int, warmup: int) -> dict:
    """The pages' levers on the current kernels, each on the same workload and
    timing: graph replay vs per-token host launches, the fused five-kernel
    layer vs the ten per-op kernels, and the null-kernel graph (every launch
    kept, every body empty: the boundary cost per token)."""
    from transformer_layer_amd import lib as L
    modes = [("fused-graph", 0, False), ("fused-eager", 0, True), ("unfused-graph", L.DEC_UNFUSED, False),
             ("null-kernels-graph", L.DEC_NULL_KERNELS, False), ("null-kernels-unfused-graph",
                                                                  L.DEC_NULL_KERNELS | L.DEC_UNFUSED, False)]
    out = {}
    for name, flags, eager in modes:
        w = Workload(cfg, flags=flags, eager=eager)
        runs = [w.timed(steps, warmup if r == 0 else 2)[0] / steps for r in range(3)]
        w.close()
        ms = float(np.median(runs))
        out[name] = {"ms_per_token": round(ms, 4), "tok_s": round(1e3 / ms, 2),
                     "runs_ms": [round(v, 4) for v in runs]}
        log(f"{name}: {ms:.4f} ms/token")
    nl = cfg.n_layers
    per_tok = {"fused": 2 + 5 * nl, "unfused": 2 + 10 * nl}
    out["dispatches_per_token"] = per_tok
    out["boundary_us"] = round(out["null-kernels-graph"]["ms_per_token"] * 1e3 / per_tok["fused"], 3)
    out["fusion_speedup"] = round(out["unfused-graph"]["ms_per_token"] / out["fused-graph"]["ms_per_token"], 4)
    out["graph_speedup"] = round(out["fused-eager"]["ms_per_token"] / out["fused-graph"]["ms_per_token"], 4)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="C4",
                    help="workload: NAME, NAME:i8 (over an int8 KV cache), NAME@CTX (CTX cached positions)")
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--null-kernels", action="store_true")
    ap.add_argument("--fuse-down", action="store_true",
                    help="4-bit weights: the gated FFN and the down projection as one kernel (four per layer)")
    ap.add_argument("--attn-chunk", type=int, default=0)
    ap.add_argument("--attn-kernel", choices=["auto", "batched", "stream", "local"], default="auto",
                    help="attention kernel (default: the library's choice for the shape)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-head", action="store_true", help="skip the greedy (LM head) timing")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of --steps tokens for the median (the first is the headline value)")
    ap.add_argument("--others", default="C3,C5,C2,C4:i8,C5:i8",
                    help="other workloads timed the same way and reported under `workloads` ('' for none); "
                         "NAME:i8 is NAME over an int8 KV cache")
    ap.add_argument("--ab", action="store_true",
                    help="only the paired A/B modes (graph/eager, fused/unfused, null kernels) on --config")
    ap.add_argument("--ffn-reps", type=int, default=4,
                    help="back-to-back sweeps over the layers when timing the gated-FFN kernel")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); "
              "the multi-GPU sharding is a design note, not a runnable path", file=sys.stderr)
        return 2

    import torch
    import synth
    from transformer_layer_amd import lib as L

    cfg = workload_config(args.config)
    if args.ab:
        res = ab_modes(cfg, args.steps, args.warmup)
        print(json.dumps({"config": cfg.name, "steps": args.steps, "ab": res}), flush=True)
        return 0
    flags = ((L.DEC_UNFUSED if args.unfused else 0) | (L.DEC_NULL_KERNELS if args.null_kernels else 0)
             | (L.DEC_FUSE_DOWN if args.fuse_down else 0)
             | {"auto": 0, "batched": L.DEC_ATTN_BATCHED, "stream": L.DEC_ATTN_STREAM,
                "local": L.DEC_ATTN_LOCAL}[args.attn_kernel])
    log(f"config {cfg.name}: building stack ({cfg.n_layers} layers)")
    w = Workload(cfg, flags, args.attn_chunk, eager=args.eager)
    st = w.st
    log(f"timing {args.steps} steps")
    ms, wall = w.timed(args.steps, args.warmup)
    err = st.check_err()
    if err:
        log(f"device error word {err:#x}")
        return 1
    tok_s = args.steps / (ms * 1e-3)
    bpt = timed_token_bytes(cfg, args.steps)
    gbs = bpt * tok_s / 1e9
    log(f"{tok_s:.1f} tok/s, {ms / args.steps:.3f} ms/token, {gbs:.0f} GB/s")
    reps = [tok_s]
    for _ in range(max(0, args.repeats - 1)):
        reps.append(args.steps / (w.timed(args.steps, 2)[0] * 1e-3))
    log(f"repeat runs: {', '.join(f'{v:.1f}' for v in reps)} tok/s")
    lo, hi = w.lo, w.hi

    head = None
    if not args.null_kernels and not args.no_head:
        head = head_timing(st, cfg, lo, hi, args.steps, args.warmup)

    roof = None
    if not args.null_kernels:
        w.reset()
        t_ffn, n_ffn, t_ffn_host = ffn_kernel_time(st, cfg, args.ffn_reps)
        ffn_bytes = synth.layer_weight_bytes(cfg)["ffn"]
        ach = ffn_bytes / t_ffn / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(cfg),
                "kernel": "dec_gated_ffn (RMSNorm + gate/up GEMV + SwiGLU)",
                "bytes_per_launch": int(ffn_bytes), "launches_timed": n_ffn,
                "avg_launch_us": round(t_ffn * 1e6, 2), "timing": "graph-replayed sweep, HIP events",
                "host_launched_avg_us": round(t_ffn_host * 1e6, 2)}
        log(f"gated FFN: {t_ffn * 1e6:.1f} us/launch, {ach:.0f} GB/s")
    w.close()
    del st

    if args.calib_copy:
        calib_copy(args.calib_copy)

    others = {}
    if not args.null_kernels and not args.unfused and not args.eager:
        for spec in [n for n in args.others.split(",") if n and n != args.config]:
            others[workload_config(spec).name] = other_workload(spec, args.steps, args.warmup, 3)

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle sample)")
        cpu = cpu_baseline(cfg)
        log(f"oracle: {cpu['value']:.4f} tok/s")

    out = {
        "metric": "batch-1 decode tok/s + achieved HBM GB/s vs peak, 7B/9B-shaped stack",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "hidden": cfg.hidden,
                   "heads_q_kv": [cfg.n_q_heads, cfg.n_kv_heads], "head_dim": cfg.head_dim,
                   "ffn": cfg.ffn, "weights": cfg.wtype, "kv_cache": cfg.kvtype,
                   "context": cfg.ctx, "decode_window": cfg.steps, "batch": 1,
                   "mode": ("unfused" if args.unfused else "fused") + ("-down" if args.fuse_down else "")
                           + ("-eager" if args.eager else "-graph") + ("-null" if args.null_kernels else ""),
                   "kernels_per_layer": 10 if args.unfused else 4 if args.fuse_down else 5,
                   "attention": args.attn_kernel, "attn_chunk": args.attn_chunk or "auto"},
        "bytes_per_token": int(bpt),
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "target_70pct_tok_s": round(0.7 * PEAK_HBM_GBS * 1e9 / bpt, 1),
        "repeat_runs": {"tok_s": [round(v, 2) for v in reps], "median": round(float(np.median(reps)), 2)},
        "wall_s_timed": round(wall, 3),
        "gpu_clocks": gpu_clocks(),
        "roofline": roof,
        "cpu_baseline": cpu,
        "with_head": head,
        "workloads": others,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
