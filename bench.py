#!/usr/bin/env python3
"""Decode-step benchmark of the quantized MoE layer on one MI355X.

One step = one decode token (or one batch of tokens for the batch config)
through every layer of the workload: route -> expert FFN (kernel A, kernel B,
shared experts) -> tail, for each layer in order on one stream; with one token
per step each layer is the fused single-launch moe_decode_layer (the
three-call path is timed beside it for comparison).  Each distinct token's
step is captured once into a HIP graph (torch.cuda.CUDAGraph over the
library's launches) and replayed; all inputs and weights are resident in HBM
before the timed region starts.

Throughput is expert-weight bytes per second: the packed codes plus scales
and biases of every expert the step touches (each touched expert counted
once per layer), divided by wall time.  Tokens/s is reported beside it.

The timed region is K back-to-back graph replays bracketed by device
synchronisation; one replay moves ~1 GB on the default workload, so the
launch/sync overhead of the bracket is far below 2% (the amortisation check
re-times K/2 steps and reports the per-step ratio).

Extra fields:
  roofline      the dominant kernel against the 8 TB/s HBM peak: its
                algorithmic bytes per launch divided by its average launch
                duration.  Fused path: the layer kernel is the only kernel of
                the step, so its average duration is the timed region over
                the launches in it (HIP events on the replay stream); bytes are
                the touched experts' weights plus the router matrix.
                Three-call path: kernel A alone, from HIP events around graph
                replays of its launches over the same layers and tokens.
  cpu_baseline  the CPU oracle (fp64, all host cores) on a bounded sample of
                the same workload, in the same unit.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
COUNTERS = os.path.join(ROOT, "profiles", "layer_kernel_qwen3_30b_a3b_48L_counters.json")
FUSED_KERNEL = "moe::layer_kernel"
COPY_KERNEL = "MulFunctor"


# the files the fused layer kernel is built from (sources, public header, flags)
LAYER_KERNEL_FILES = ["quantized_moe_decode_amd/csrc/" + f for f in
                      ("api.hpp", "common.hpp", "qgemv.hpp", "topk.hpp", "layer_kernel.hpp", "layer.hip",
                       "layer_a4.hip", "layer_a6.hip", "layer_a8.hip",
                       "layer_a4p.hip", "layer_a6p.hip", "layer_a8p.hip")] + \
                     ["include/moe_decode.h", "quantized_moe_decode_amd/build.py"]


def kernel_sources_sha256() -> str:
    """Hash of the files the fused layer kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for rel in LAYER_KERNEL_FILES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def summarize_counters(fetch_csv: str, write_csv: str, copy_mib: int, command: str) -> dict:
    """Per-launch HBM bytes of the fused layer kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the calibration copy kernel of known size."""
    import csv
    import statistics

    def per_kernel(path, counter):
        layer, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if FUSED_KERNEL in r["Kernel_Name"]:
                layer.append(v)
            elif COPY_KERNEL in r["Kernel_Name"]:
                copy.append(v)
        if not layer or not copy:
            raise SystemExit(f"{path}: no {counter} rows for the layer kernel or the copy kernel")
        return statistics.mean(layer), len(layer), statistics.mean(copy)

    known_kib = copy_mib * 1024.0
    f_layer, n_f, f_copy = per_kernel(fetch_csv, "FETCH_SIZE")
    w_layer, n_w, w_copy = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = known_kib / f_copy, known_kib / w_copy
    return {
        "kernel": FUSED_KERNEL, "workload": "qwen3_30b_a3b_moe",
        "command": command,
        "sources_sha256": kernel_sources_sha256(),
        "fetch_kib_per_launch_raw": round(f_layer, 2), "write_kib_per_launch_raw": round(w_layer, 2),
        "launches": [n_f, n_w],
        "copy_mib": copy_mib, "copy_fetch_kib_raw": round(f_copy, 2), "copy_write_kib_raw": round(w_copy, 2),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": int(round((f_layer * f_scale + w_layer * w_scale) * 1024)),
    }


def traffic_per_launch():
    """HBM bytes per fused launch from the committed counter record, or None
    when the record is missing or the kernel sources changed since it was taken."""
    import json as _json
    try:
        rec = _json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return rec["hbm_bytes_per_launch"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="qwen3_30b_a3b_moe")
    ap.add_argument("--tokens", type=int, default=8,
                    help="distinct pre-generated tokens (or token batches) rotated over the steps")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--profile-run", action="store_true",
                    help="for counter collection: skip the comparison path and the CPU baseline, "
                         "and end with a plain copy kernel of --copy-mib MiB (the counters' calibration)")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter record from two rocprofv3 --pmc counter_collection.csv "
                         "files (FETCH_SIZE, WRITE_SIZE of a --profile-run) and exit")
    ap.add_argument("--counters-command", default="", help="the profiler command, for the record")
    ap.add_argument("--ws", choices=("shared", "per-layer"), default="shared",
                    help="fused path: one workspace for all layers of a step (default) or one per layer")
    ap.add_argument("--path", choices=("fused", "three-call"), default=None,
                    help="fused single-launch layer (default for one token per step) or "
                         "route + expert FFN + tail (default for several tokens per step)")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_counters:
        rec = summarize_counters(*args.summarize_counters, args.copy_mib, args.counters_command)
        with open(COUNTERS, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MoE decode layer here runs on a single MI355X "
              "and has no multi-GPU path (the sharding design is described in DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import quantized_moe_decode_amd as qmd
    from quantized_moe_decode_amd.layer import layer_from_host, share_fused_workspace, tensor_from_encoded

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = mi.CONFIGS[args.config]
    L = args.layers or cfg.n_layers
    T = cfg.n_tokens
    R = args.tokens

    # ---- weights and inputs, resident in HBM
    t0 = time.time()
    layers, host_keep = [], {}
    if args.profile_run:
        args.no_cpu_baseline = True
    keep_for_cpu = 0 if args.no_cpu_baseline else min(L, 4)
    for li in range(L):
        w = mi.gen_layer_weights(cfg, li)
        layers.append(layer_from_host(cfg, w, dev, n_tokens=T))
        if li < keep_for_cpu:
            host_keep[li] = w
        if li % 8 == 7 or li == L - 1:
            log(f"[bench] {li + 1}/{L} layers resident ({time.time() - t0:.1f}s)")
    xs = [[None] * L for _ in range(R)]
    rs = [[None] * L for _ in range(R)]
    host_tok = {}
    for r in range(R):
        for li in range(L):
            tok = [mi.gen_token(cfg, li, r * T + t) for t in range(T)]
            x = np.stack([a for a, _ in tok])
            rd = np.stack([b for _, b in tok])
            if li < keep_for_cpu and r == 0:
                host_tok[li] = (x, rd)
            xs[r][li] = tensor_from_encoded(x, cfg.x_dtype, dev)
            rs[r][li] = tensor_from_encoded(rd, cfg.resid_dtype, dev)
    outs = [torch.zeros(T, cfg.d_in, device=dev) for _ in range(L)]
    if args.ws == "shared":
        share_fused_workspace(layers)
    torch.cuda.synchronize()

    path = args.path or ("fused" if T == 1 else "three-call")
    if path == "fused" and T != 1:
        print("the fused layer launch takes one token per step", file=sys.stderr)
        sys.exit(2)

    def step_eager(r, which=None):
        fused = (which or path) == "fused"
        for li in range(L):
            if fused:
                layers[li].forward_fused(xs[r][li], rs[r][li], outs[li])
            else:
                layers[li].forward(xs[r][li], rs[r][li], outs[li])

    # ---- capture one graph per distinct token
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(R):
            step_eager(r)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_eager(r)
        graphs.append(g)
    torch.cuda.synchronize()

    # ---- expert bytes per step (touched experts, each once per layer)
    per_expert = layers[0].gate.nbytes() + layers[0].up.nbytes() + layers[0].down.nbytes()
    shared_bytes = 0
    if layers[0].shared is not None:
        shared_bytes = sum(sq.nbytes(layers[0].n_shared) for sq in layers[0].shared)
    step_bytes, step_touched = [], []
    for r in range(R):
        graphs[r].replay()
        torch.cuda.synchronize()
        touched = 0
        for li in range(L):
            ids = layers[li].ids.cpu().numpy()
            touched += len(set(int(e) for e in ids.reshape(-1) if 0 <= e < cfg.n_experts))
        step_touched.append(touched)
        step_bytes.append(touched * per_expert + L * shared_bytes)

    # ---- timed region
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()

    def timed(nsteps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(nsteps):
            graphs[i % R].replay()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1000.0

    wall0 = time.perf_counter()
    secs = timed(args.steps)
    wall = time.perf_counter() - wall0
    bytes_total = sum(step_bytes[i % R] for i in range(args.steps))
    gbps = bytes_total / secs / 1e9
    tok_s = args.steps * T / secs
    half = max(1, args.steps // 2)
    secs_half = timed(half)
    amort = (secs_half / half) / (secs / args.steps)

    # ---- roofline of the dominant kernel.  With the fused path every launch of
    # the step is the layer kernel, so its average launch duration is the timed
    # region divided by the launches in it; algorithmic bytes per launch are
    # the touched experts' weights plus the router matrix.
    router_bytes = layers[0].router.numel() * layers[0].router.element_size()
    if path == "fused":
        launches = args.steps * L
        avg_us = secs / launches * 1e6
        alg = (bytes_total + args.steps * L * router_bytes) / launches
        roofline = {"kernel": "layer_kernel (route + kernel A + kernel B + tail, one launch per layer)",
                    "bound": "hbm", "achieved": round(alg / (avg_us * 1e-6) / 1e9, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(alg / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "traffic": traffic_per_launch(), "traffic_unit": "HBM bytes per launch",
                    "avg_launch_us": round(avg_us, 3),
                    "bytes_per_launch": int(alg)}
    else:
        # kernel A alone, from graphs holding only its launches for the same tokens
        a_graphs, a_bytes = [], []
        for r in range(R):
            graphs[r].replay()           # leaves token r's expert ids in every layer
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for li in range(L):
                    lay = layers[li]
                    qmd.moe_decode_gate_up(xs[r][li], lay.gate, lay.up, lay.ids, lay.act, lay.ffn_ws)
            a_graphs.append(g)
            a_bytes.append(step_touched[r] * (layers[0].gate.nbytes() + layers[0].up.nbytes()))
        for g in a_graphs:
            g.replay()
        torch.cuda.synchronize()
        reps = max(4, args.steps // 4)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(reps):
            a_graphs[i % R].replay()
        ev1.record()
        torch.cuda.synchronize()
        a_secs = ev0.elapsed_time(ev1) / 1000.0
        launches = reps * L
        a_total = sum(a_bytes[i % R] for i in range(reps))
        achieved = a_total / a_secs / 1e9
        roofline = {"kernel": "gate_up_kernel (kernel A: gate/up GEMV + SwiGLU)",
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                    "avg_launch_us": round(a_secs / launches * 1e6, 3),
                    "bytes_per_launch": int(a_total / launches)}

    # ---- the other path on the same tokens, for comparison (not the headline)
    other = None
    if T == 1 and not args.profile_run:
        which = "three-call" if path == "fused" else "fused"
        og = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_eager(r, which)
            og.append(g)
        for g in og:
            g.replay()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        n_o = max(10, args.steps // 3)
        ev0.record()
        for i in range(n_o):
            og[i % R].replay()
        ev1.record()
        torch.cuda.synchronize()
        o_secs = ev0.elapsed_time(ev1) / 1000.0
        other = {"path": which, "GBps": round(sum(step_bytes[i % R] for i in range(n_o)) / o_secs / 1e9, 2),
                 "ms_per_step": round(o_secs / n_o * 1e3, 4)}

    # ---- practical ceiling: the library's streaming-read probe on cold data, one
    # layer's worth of expert bytes per launch and 1 GiB per launch, each launch
    # on a different slice of a 4 GiB buffer (well beyond the 256 MB last-level
    # cache); launches captured in a graph and timed with HIP events.
    ceiling = None
    if not args.no_ceiling and not args.profile_run:
        big = torch.ones((4 << 30) // 4, device=dev)
        ceiling = {"kernel": "read_probe_kernel (moe_decode_read_probe: 16-byte loads, read once)"}
        for label, nbytes in (("per_layer_expert_bytes", int(np.mean(step_bytes)) // L // 16 * 16),
                              ("1GiB", 1 << 30)):
            nel = nbytes // 4
            nsl = big.numel() // nel
            reps = min(64, nsl)
            sl = [big[(i % nsl) * nel:(i % nsl + 1) * nel] for i in range(reps)]
            part = torch.zeros(qmd.read_probe_blocks(nbytes), device=dev)
            ss = torch.cuda.Stream()
            ss.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(ss):
                for i in range(reps):
                    qmd.moe_decode_read_probe(sl[i], part)
            torch.cuda.current_stream().wait_stream(ss)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    qmd.moe_decode_read_probe(sl[i], part)
            g.replay()
            torch.cuda.synchronize()
            assert float(part.sum().item()) == float(nel), "read probe did not read every byte once"
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            g.replay()
            g.replay()
            ev1.record()
            torch.cuda.synchronize()
            t = ev0.elapsed_time(ev1) / 1000.0 / (2 * reps)
            ceiling[label] = {"bytes": nbytes, "us_per_launch": round(t * 1e6, 3),
                              "GBps": round(nbytes / t / 1e9, 1)}
        del big
        torch.cuda.synchronize()

    # ---- CPU oracle baseline on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = oracle.num_threads()
        done_layers, cpu_bytes = 0, 0
        c0 = time.perf_counter()
        li = 0
        while time.perf_counter() - c0 < args.cpu_seconds:
            k = li % keep_for_cpu
            x, rd = host_tok[k]
            res = oracle.layer(cfg, host_keep[k], x, rd)
            touched = len(set(int(e) for e in res["route"]["ids"].reshape(-1)))
            cpu_bytes += touched * per_expert + shared_bytes
            done_layers += 1
            li += 1
        csecs = time.perf_counter() - c0
        cpu = {"value": round(cpu_bytes / csecs / 1e9, 4), "unit": "GB/s", "cores": nthreads,
               "kind": "oracle",
               "tokens_per_s": round(done_layers / L * T / csecs, 4),
               "sample": f"{done_layers} layer evaluations of the first {keep_for_cpu} layers "
                         f"(token 0), {csecs:.1f}s, fp64, OpenMP over output rows"}

    copy = None
    if args.profile_run:
        # a plain copy of known size: reads and writes copy-mib MiB each, so the
        # HBM counters of a profiler run can be scaled to bytes
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        copy = {"kernel": "elementwise mul by 1 (torch)", "bytes_read": n * 4, "bytes_written": n * 4,
                "launches": 3}

    line = {
        "metric": "expert-weight HBM GB/s (% of ~8 TB/s) and MoE-layer decode tokens/s",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(secs / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 weights, f32 accumulation" if cfg.bits_gate_up == 4 else
                 f"u{cfg.bits_gate_up}/u{cfg.bits_down} weights, f32 accumulation",
        "data": "synthetic (seeded generator; random-init weights of the stated shapes)",
        "config": {"workload": cfg.name, "layers": L, "tokens_per_step": T,
                   "d_in": cfg.d_in, "d_ff": cfg.d_ff, "experts": cfg.n_experts,
                   "top_k": cfg.top_k, "bits": [cfg.bits_gate_up, cfg.bits_down],
                   "distinct_tokens": R, "parallelism": "single GPU"},
        "tokens_per_s": round(tok_s, 2),
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "expert_bytes_per_step": int(np.mean(step_bytes)),
        "amortisation_ratio_half_vs_full": round(amort, 4),
        "wall_s_timed": round(wall, 4),
        "path": path,
        "other_path": other,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ceiling": ceiling,
    }
    if copy is not None:
        line["calibration_copy"] = copy
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    main()
