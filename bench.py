#!/usr/bin/env python3
"""Decode-step benchmark of the quantized MoE layer on one MI355X.

One step = one decode token (or one batch of 32 tokens) through every layer of
a workload, layers in order on one stream: route -> expert FFN (kernel A,
kernel B, shared experts) -> tail, which with one token per step is the
single fused moe_decode_layer launch per layer (the three-call path is timed
beside it).  Each distinct token's step is captured once into a HIP graph
(quantized_moe_decode_amd.layer.DecodeStep) and replayed; weights and inputs
are resident in HBM before any timing starts.

Every workload is measured (headline: the Qwen3-30B-A3B-shaped layer, 48
layers, one token per step); `--config NAME` measures one.

Throughput is expert-weight bytes per second: the packed codes plus scales
and biases of every expert a step touches (each touched expert once per
layer), divided by wall time; tokens/s beside it.  Router, act, partial, x,
residual and output bytes are reported as other bytes.

Sample protocol (the pages' amortisation lesson: per-call overhead in a
timed region manufactures wins and losses):
  * the host round trip of an empty graph launch plus synchronisation, o, is
    measured first;
  * a sample is n step replays between two HIP events on the replay stream,
    bracketed by device synchronisation, with n large enough that o is under
    2% of the sample, that the sample moves at least --bytes-per-sample bytes
    of expert weight and lasts at least --min-sample-ms;
  * --samples samples (at least 10) give the median, min and max; the
    per-step time of a sample of 2n steps must agree with the median within
    2% (amortisation_ratio_2n);
  * after the samples every launch's workspace error word must be clear.

Extra fields per workload:
  roofline      the dominant kernel against the 8 TB/s HBM peak: algorithmic
                expert bytes per launch over its average launch duration (HIP
                events around graph replays of that kernel's launches only,
                or, on the fused path, the step itself, whose launches are all
                that kernel); traffic = HBM bytes per launch from the committed
                rocprofv3 counter record, when the kernel sources are the ones
                it was taken with.
  cpu_baseline  the CPU oracle (fp64) on a bounded sample of the same workload
                and tokens, all host threads and one thread, with the CPU
                model.  The oracle's results of that sample are also the check
                of the GPU's: one replay's outputs of every layer (the first
                tokens of a batch) must match within 2e-3 of their infinity
                norm, expert ids exactly where the routing margin holds
                (`validated`).  A failed check prints no value and exits 1.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
HEADLINE = "qwen3_30b_a3b_moe"
# the 32- and 256-token workloads right after the headline: they run on the headline's device weights
ALL_CONFIGS = [HEADLINE, "qwen3_30b_a3b_moe_batch32", "qwen3_30b_a3b_moe_prefill256", "tiny_e8_top2",
               "qwen1.5_moe_a2.7b", "dots_llm1_mixed_bit"]
FUSED_KERNEL = "moe::layer_kernel"
BATCH_GATE_UP_KERNEL = "moe::gate_up_batch_q4"
GROUPED_FFN_KERNEL = "moe::ffn_grouped_fused"        # gate/up and down units of the grouped call, one launch
GROUPED_BUCKET_KERNEL = "moe::grouped_bucket_kernel"
MAX_DECODE_TOKENS = 32          # above this the layer takes the grouped (matrix-core) expert FFN
COPY_KERNEL = "MulFunctor"
TOL = 2e-3
MARGIN = 1e-3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------- counter records
def kernel_sources_sha256() -> str:
    """Hash of every file the library is built from (sources, public header, build script)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_decode_amd", "csrc")
    files = sorted(os.path.join("quantized_moe_decode_amd", "csrc", f) for f in os.listdir(csrc))
    files += ["include/moe_decode.h", "quantized_moe_decode_amd/build.py"]
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def counters_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"counters_{workload}.json")


def dominant_kernel(cfg) -> str:
    if cfg.n_tokens == 1:
        return FUSED_KERNEL
    return BATCH_GATE_UP_KERNEL if cfg.n_tokens <= MAX_DECODE_TOKENS else GROUPED_FFN_KERNEL


def unit_kernels(cfg) -> list:
    """The kernels of the roofline unit: the dominant kernel, or for the
    grouped path the two launches of one grouped expert FFN call (bucketing,
    then gate/up and down units in one launch)."""
    k = dominant_kernel(cfg)
    return [GROUPED_BUCKET_KERNEL, k] if k == GROUPED_FFN_KERNEL else [k]


def summarize_counters(fetch_csv, write_csv, workload, copy_mib, command) -> dict:
    """Per-launch HBM bytes of the workload's roofline unit from two rocprofv3
    --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what
    the same counter reads for the calibration copy kernel of known size (a
    unit of several kernels: the sum of their per-dispatch means)."""
    import csv
    import moe_inputs as mi
    kernels = unit_kernels(mi.CONFIGS[workload])
    kernel = " + ".join(kernels)

    def per_kernel(path, counter):
        k, copy = {n: [] for n in kernels}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            for n in kernels:
                if n in r["Kernel_Name"]:
                    k[n].append(v)
            if COPY_KERNEL in r["Kernel_Name"]:
                copy.append(v)
        if not all(k.values()) or not copy:
            raise SystemExit(f"{path}: no {counter} rows for {kernel} or the copy kernel")
        return sum(statistics.mean(v) for v in k.values()), min(len(v) for v in k.values()), statistics.mean(copy)

    known_kib = copy_mib * 1024.0
    f_k, n_f, f_copy = per_kernel(fetch_csv, "FETCH_SIZE")
    w_k, n_w, w_copy = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = known_kib / f_copy, known_kib / w_copy
    return {
        "kernel": kernel, "workload": workload, "command": command,
        "sources_sha256": kernel_sources_sha256(),
        "fetch_kib_per_launch_raw": round(f_k, 2), "write_kib_per_launch_raw": round(w_k, 2),
        "launches": [n_f, n_w],
        "copy_mib": copy_mib, "copy_fetch_kib_raw": round(f_copy, 2), "copy_write_kib_raw": round(w_copy, 2),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": int(round((f_k * f_scale + w_k * w_scale) * 1024)),
    }


def traffic_per_launch(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    record, or None when there is none or the sources changed since."""
    try:
        rec = json.load(open(counters_path(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return rec["hbm_bytes_per_launch"]


# --------------------------------------------------------------- host state
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_SMI_HELPER = r"""
import json, subprocess, sys
for _ in sys.stdin:
    out = {}
    for key, args in (("metric", ["metric", "-g", "0", "--usage", "--clock", "--json"]),
                      ("process", ["process", "-g", "0", "--json"])):
        try:
            r = subprocess.run(["amd-smi", *args], capture_output=True, text=True, timeout=20)
            out[key] = json.loads(r.stdout) if r.returncode == 0 else None
        except Exception:
            out[key] = None
    print(json.dumps(out), flush=True)
"""


class GpuStateSampler:
    """amd-smi's view of GPU 0 (busy percentages, clocks, other processes),
    sampled on request by a helper process started before this process
    touches the GPU: a process that has initialised the GPU must not start
    other programs itself.  A contended GPU invalidates timings."""

    def __init__(self):
        try:
            self.proc = subprocess.Popen([sys.executable, "-c", _SMI_HELPER], stdin=subprocess.PIPE,
                                         stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            self.proc = None

    def sample(self) -> dict:
        state = {"gfx_busy_pct": None, "umc_busy_pct": None, "gfx_clk_mhz_max": None, "mem_clk_mhz": None,
                 "other_processes": None}
        if self.proc is None:
            return state
        try:
            self.proc.stdin.write("s\n")
            self.proc.stdin.flush()
            out = json.loads(self.proc.stdout.readline())
        except (OSError, ValueError):
            return state
        try:
            m = out["metric"]
            m = (m["gpu_data"] if isinstance(m, dict) else m)[0]
            state["gfx_busy_pct"] = m["usage"]["gfx_activity"]["value"]
            state["umc_busy_pct"] = m["usage"]["umc_activity"]["value"]
            clk = m["clock"]
            gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
            state["gfx_clk_mhz_max"] = max(x for x in gfx if isinstance(x, (int, float)))
            mem = [v["clk"]["value"] for k, v in clk.items() if k.startswith("mem_") and isinstance(v, dict)]
            state["mem_clk_mhz"] = mem[0] if mem else None
        except (KeyError, TypeError, IndexError, ValueError):
            pass
        try:
            p = out["process"]
            p = (p["gpu_data"] if isinstance(p, dict) and "gpu_data" in p else p)[0]
            procs = [q.get("process_info") for q in p.get("process_list", []) if isinstance(q, dict)]
            state["gpu_processes"] = len([q for q in procs if isinstance(q, dict)])
            state["other_processes"] = len([q for q in procs if isinstance(q, dict) and q.get("pid") != os.getpid()])
        except (KeyError, TypeError, AttributeError, IndexError):
            pass
        return state

    def close(self):
        if self.proc is not None:
            try:
                self.proc.stdin.close()
                self.proc.wait(timeout=30)
            except (OSError, subprocess.SubprocessError):
                self.proc.kill()


# ------------------------------------------------------------------ helpers
def state_sampler(profile_run: bool):
    """The amd-smi helper, started before anything touches the GPU; a profile
    run starts none: under rocprofv3 the profiler has initialised the GPU
    before this program runs, and a process that has must not start others."""
    return None if profile_run else GpuStateSampler()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref)) / scale) if scale else float(np.max(np.abs(got - ref)))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300,
                    help="headline: at least this many timed steps over all samples")
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="after the warm-up steps, keep replaying for at least this long before timing")
    ap.add_argument("--samples", type=int, default=10)
    ap.add_argument("--config", default="all", help="a workload name, or 'all'")
    ap.add_argument("--tokens", type=int, default=8,
                    help="distinct pre-generated tokens (or token batches) rotated over the steps")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--steps-per-graph", type=int, default=0,
                    help="steps captured per graph replay (0: 32 for a one-layer workload, whose step is "
                         "shorter than the host's graph launch, else 1)")
    ap.add_argument("--expert-path", choices=["auto", "decode", "grouped"], default="auto",
                    help="expert FFN of a multi-token step: the decode kernels (up to 32 tokens), the "
                         "grouped matrix-core call, or auto (grouped above 32 tokens)")
    ap.add_argument("--bytes-per-sample", type=float, default=1e9,
                    help="minimum expert-weight bytes per timed sample (lower it to see the amortisation trap)")
    ap.add_argument("--min-sample-ms", type=float, default=20.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle time, all threads, on the headline workload (a third of it on the others)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (and with it the check of the outputs)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--profile-run", action="store_true",
                    help="for counter collection: one workload, a few steps, no comparison or CPU leg, "
                         "then a plain copy kernel of --copy-mib MiB (the counters' calibration)")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter record of --config from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE of a --profile-run)")
    ap.add_argument("--counters-command", default="", help="the profiler command, for the record")
    return ap.parse_args()


# ------------------------------------------------------------ one workload
class Workload:
    """Device layers, tokens and the captured step of one workload."""

    def __init__(self, cfg, n_layers, n_distinct, dev, stacks=None, grouped=None, repeat=1):
        import torch
        import moe_inputs as mi
        from quantized_moe_decode_amd.layer import (DecodeLayer, DecodeStep, stack_to_device,
                                                    tensor_from_encoded)
        self.cfg, self.L, self.R, self.T = cfg, n_layers, n_distinct, cfg.n_tokens
        t0 = time.time()
        if stacks is None:
            stacks = []
            for li in range(n_layers):
                w = mi.gen_layer_weights(cfg, li)
                router = tensor_from_encoded(w["router"], cfg.router_dtype, dev)
                g, u, d = (stack_to_device(w[p], dev) for p in ("gate", "up", "down"))
                sh = ([stack_to_device(w[p], dev) for p in ("shared_gate_proj", "shared_up", "shared_down")]
                      if cfg.n_shared else None)
                wg = tensor_from_encoded(w["shared_gate_w"], "bf16", dev) if cfg.shared_gate else None
                stacks.append((router, g, u, d, sh, wg))
                del w
                if li % 12 == 11 or li == n_layers - 1:
                    log(f"[bench] {cfg.name}: {li + 1}/{n_layers} layers resident ({time.time() - t0:.1f}s)")
        self.stacks = stacks
        self.layers = [DecodeLayer(s[0], cfg.top_k, cfg.renormalize, s[1], s[2], s[3], s[4], s[5], self.T,
                                   grouped=grouped) for s in stacks]
        # token r of layer l: x and resid for tokens r*T .. r*T+T-1 (first draw of each)
        self.host_x, self.host_r = [], []
        xs, rs = [], []
        for r in range(n_distinct):
            hx, hr, dx, dr = [], [], [], []
            for li in range(n_layers):
                tok = [mi.gen_token(cfg, li, r * self.T + t) for t in range(self.T)]
                x = np.stack([a for a, _ in tok])
                res = np.stack([b for _, b in tok])
                hx.append(x)
                hr.append(res)
                dx.append(tensor_from_encoded(x, cfg.x_dtype, dev))
                dr.append(tensor_from_encoded(res, cfg.resid_dtype, dev))
            self.host_x.append(hx)
            self.host_r.append(hr)
            xs.append(dx)
            rs.append(dr)
        self.path = "fused" if self.T == 1 else "three-call"
        self.step = DecodeStep(self.layers, xs, rs, path=self.path, repeat=repeat)
        self.step.capture()
        g0 = self.layers[0]
        self.per_expert = g0.gate.nbytes() + g0.up.nbytes() + g0.down.nbytes()
        self.shared_bytes = sum(sq.nbytes(g0.n_shared) for sq in g0.shared) if g0.shared is not None else 0
        self.router_bytes = g0.router.numel() * g0.router.element_size()
        # expert bytes per distinct step: touched experts (each once per layer) + shared
        self.step_bytes, self.step_touched = [], []
        for r in range(n_distinct):
            self.step.replay(r)
            torch.cuda.synchronize()
            touched = 0
            for lay in self.layers:
                ids = lay.ids.cpu().numpy()
                touched += len(set(int(e) for e in ids.reshape(-1) if 0 <= e < cfg.n_experts))
            self.step_touched.append(touched)
            self.step_bytes.append(touched * self.per_expert + n_layers * self.shared_bytes)
        torch.cuda.synchronize()

    def other_bytes_per_step(self) -> int:
        """Router matrix, x, residual, out, act and partial (written and read) per step."""
        cfg, T, L = self.cfg, self.T, self.L
        el = {"f32": 4, "f16": 2, "bf16": 2}
        per_layer = (self.router_bytes + T * cfg.d_in * (el[cfg.x_dtype] + el[cfg.resid_dtype] + 4)
                     + 2 * T * (cfg.top_k + cfg.n_shared) * (cfg.d_ff_shared or cfg.d_ff + cfg.d_in) * 4)
        return per_layer * L


def timed_replays(step, n, R, offset=0):
    """Seconds for n back-to-back step replays (HIP events on the replay stream,
    device synchronisation on both sides)."""
    import torch
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        step.replay((offset + i) % R)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1000.0


def round_trip_overhead() -> float:
    """Median host seconds of launching a one-kernel graph and synchronising."""
    import torch
    x = torch.zeros(1, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        x.add_(1.0)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        x.add_(1.0)
    torch.cuda.synchronize()
    ts = []
    for _ in range(30):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts[5:])


def measure(wl, args, overhead, min_steps=0):
    """The sample protocol: n sized from the round trip, the sample bytes and
    duration; >= args.samples samples; a 2n sample for the amortisation check."""
    R, rep = wl.R, wl.step.repeat                  # one replay = rep steps
    for i in range(args.warmup):
        wl.step.replay(i % R)
    # and at least --warmup-ms of replays, so that the clocks have left their
    # idle state before a short step is timed
    t_end = time.perf_counter() + args.warmup_ms * 1e-3
    while time.perf_counter() < t_end:
        timed_replays(wl.step, 4 * R, R)
    pilot = timed_replays(wl.step, max(3, R), R) / max(3, R)    # per replay
    mean_bytes = float(np.mean(wl.step_bytes))
    n = max(1, int(np.ceil(50.0 * overhead / pilot)),            # round trip < 2% of a sample
            int(np.ceil(args.bytes_per_sample / (mean_bytes * rep))),   # >= bytes_per_sample per sample
            int(np.ceil(args.min_sample_ms * 1e-3 / pilot)),
            int(np.ceil(min_steps / (args.samples * rep))))
    samples = [timed_replays(wl.step, n, R, offset=k * n) / (n * rep) for k in range(args.samples)]
    two_n = timed_replays(wl.step, 2 * n, R) / (2 * n * rep)
    med = statistics.median(samples)
    return dict(n=n * rep, samples=samples, median=med, min=min(samples), max=max(samples),
                amortisation_ratio_2n=two_n / med, pilot=pilot / rep)


def step_bytes_for(wl, n, offset=0):
    return sum(wl.step_bytes[(offset + i) % wl.R] for i in range(n)) / n


def roofline_of(wl, meas, args):
    """The dominant kernel of the workload against the HBM peak."""
    import torch
    import quantized_moe_decode_amd as qmd
    cfg, L, R = wl.cfg, wl.L, wl.R
    if wl.path == "fused":
        # every launch of the step is the layer kernel: its average duration is
        # the step time over the launches in it
        avg_s = meas["median"] / L
        alg = float(np.mean(wl.step_bytes)) / L
        name = "layer_kernel (route + kernel A + kernel B + tail, one launch per layer)"
    else:
        # kernel A (multi-token gate/up) alone, or for the grouped path the
        # grouped expert FFN call (its bucketing, gate/up and down launches):
        # graphs of those launches only, for the same layers and tokens (each
        # layer's ids left by a replay of the step)
        graphs, a_bytes = [], []
        grouped = wl.layers[0].grouped
        per_unit = (wl.per_expert if grouped else wl.layers[0].gate.nbytes() + wl.layers[0].up.nbytes())
        for r in range(R):
            wl.step.replay(r)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for li, lay in enumerate(wl.layers):
                    if grouped:
                        qmd.moe_decode_expert_ffn_grouped(wl.step.xs[r][li], lay.gate, lay.up, lay.down, lay.ids,
                                                          lay.scores, lay.act, lay.partial, lay.ffn_ws)
                    else:
                        qmd.moe_decode_gate_up(wl.step.xs[r][li], lay.gate, lay.up, lay.ids, lay.act, lay.ffn_ws)
            graphs.append(g)
            a_bytes.append(wl.step_touched[r] * per_unit)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        reps = max(8, 4 * R)
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            graphs[i % R].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        avg_s = e0.elapsed_time(e1) / 1000.0 / (reps * L)
        alg = sum(a_bytes[i % R] for i in range(reps)) / (reps * L)
        name = ("expert_ffn_grouped (bucketing + ffn_grouped_fused: the matrix-core expert FFN "
                "of every touched expert, per layer)" if grouped else
                "gate_up_batch_q4 (kernel A: gate/up GEMV + SwiGLU for every token of a touched expert)")
        del graphs
    achieved = alg / avg_s / 1e9
    traffic = traffic_per_launch(cfg.name)
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "avg_launch_us": round(avg_s * 1e6, 3), "bytes_per_launch": int(alg),
            "bytes_counted": "expert weights (codes, scales, biases) of the touched experts"}


def other_path(wl, args):
    """The three-call path on the same tokens (one token per step), for comparison."""
    import torch
    graphs = wl.step.capture(path="three-call")
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    n = max(10, args.steps // 3)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        graphs[i % wl.R].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1000.0 / wl.step.repeat     # one replay = repeat steps
    import quantized_moe_decode_amd as qmd
    ok = all(qmd.workspace_status(l.route_ws) == qmd.MOE_OK for l in wl.layers)
    if not ok:
        raise SystemExit(f"{wl.cfg.name}: a route wait timed out on the three-call path")
    return {"path": "three-call", "GBps": round(step_bytes_for(wl, n) * n / secs / 1e9, 2),
            "ms_per_step": round(secs / n * 1e3, 4)}


def ceiling(dev, per_layer_bytes):
    """The library's streaming-read probe on cold slices of a 4 GiB buffer: one
    layer's expert bytes per launch, and 1 GiB per launch."""
    import torch
    import quantized_moe_decode_amd as qmd
    big = torch.ones((4 << 30) // 4, device=dev)
    out = {"kernel": "read_probe_kernel (moe_decode_read_probe: 16-byte loads, read once)"}
    for label, nbytes in (("per_layer_expert_bytes", per_layer_bytes // 16 * 16), ("1GiB", 1 << 30)):
        nel = nbytes // 4
        nsl = big.numel() // nel
        reps = min(64, nsl)
        sl = [big[(i % nsl) * nel:(i % nsl + 1) * nel] for i in range(reps)]
        part = torch.zeros(qmd.read_probe_blocks(nbytes), device=dev)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(reps):
                qmd.moe_decode_read_probe(sl[i], part)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                qmd.moe_decode_read_probe(sl[i], part)
        g.replay()
        torch.cuda.synchronize()
        if float(part.sum().item()) != float(nel):
            raise SystemExit("read probe did not read every byte once")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1000.0 / (2 * reps)
        out[label] = {"bytes": nbytes, "us_per_launch": round(t * 1e6, 3), "GBps": round(nbytes / t / 1e9, 1)}
    del big
    torch.cuda.synchronize()
    return out


def cpu_leg(wl, args, seconds):
    """The oracle on a bounded sample of the workload: replay 0's tokens through
    every layer (the first 4 tokens of a batch), all host threads, timed, its
    results compared with the GPU's outputs of one replay of the same step;
    then the first layers again on one thread."""
    import torch
    import oracle
    cfg, L = wl.cfg, wl.L
    tcheck = min(wl.T, 4)
    wl.step.replay(0)
    torch.cuda.synchronize()
    gpu_out = [o.cpu().numpy()[:tcheck] for o in wl.step.outs]
    gpu_ids = [lay.ids.cpu().numpy()[:tcheck] for lay in wl.layers]
    err_words = wl.step.error_words()

    def one(li):
        """The oracle on layer li (its weight generation not timed)."""
        x, r = wl.host_x[0][li][:tcheck], wl.host_r[0][li][:tcheck]
        w, ids, scores = oracle.selected_weights(cfg, li, x)
        t0 = time.perf_counter()
        res = oracle.layer(cfg, w, x, r, ids=ids, scores=scores)
        return res, time.perf_counter() - t0

    threads = oracle.num_threads()
    secs, bytes_done, layers_done = 0.0, 0, 0
    worst = {"out": 0.0, "moe": 0.0}
    checked, near_tie_skipped, ids_mismatch = 0, 0, 0
    wall0 = time.perf_counter()
    li = 0
    while True:
        res, dt = one(li % L)
        secs += dt
        layers_done += 1
        bytes_done += len(set(res["route"]["ids"].reshape(-1).tolist())) * wl.per_expert + wl.shared_bytes
        if li < L:                                   # the check, once per layer
            logits = res["route"]["logits"]
            top = np.sort(logits, axis=1)[:, ::-1][:, :cfg.top_k + 1]
            margin = np.all(np.diff(top, axis=1) <= -MARGIN, axis=1)
            same = np.all(gpu_ids[li] == res["route"]["ids"], axis=1)
            ids_mismatch += int(np.sum(margin & ~same))
            for t in range(tcheck):
                if not same[t]:
                    near_tie_skipped += 1            # a near tie the GPU ranked differently
                    continue
                resid = oracle.decode(wl.host_r[0][li][t], cfg.resid_dtype)
                worst["out"] = max(worst["out"], rel_err(gpu_out[li][t], res["out"][t]))
                worst["moe"] = max(worst["moe"], rel_err(gpu_out[li][t] - resid, res["out"][t] - resid))
                checked += 1
        li += 1
        if li >= L and secs >= seconds:
            break
        if time.perf_counter() - wall0 > 4 * seconds + 60:
            break
    ok = err_words == 0 and ids_mismatch == 0 and checked > 0 and worst["out"] <= TOL and worst["moe"] <= TOL
    validated = {"ok": bool(ok), "layers": L, "tokens_per_layer": tcheck, "outputs_checked": checked,
                 "near_tie_skipped": near_tie_skipped, "ids_mismatch_with_margin": ids_mismatch,
                 "max_rel_err_out": worst["out"], "max_rel_err_moe_term": worst["moe"], "tol": TOL,
                 "error_words": int(err_words)}
    # one thread, the first layers
    oracle.set_num_threads(1)
    s1, b1, n1 = 0.0, 0, 0
    try:
        while s1 < seconds / 3 or n1 < 1:
            res, dt = one(n1 % L)
            s1 += dt
            b1 += len(set(res["route"]["ids"].reshape(-1).tolist())) * wl.per_expert + wl.shared_bytes
            n1 += 1
    finally:
        oracle.set_num_threads(threads)
    cpu = {"value": round(bytes_done / secs / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "tokens_per_s": round(layers_done / L * tcheck / secs, 4),
           "one_thread": {"value": round(b1 / s1 / 1e9, 4), "unit": "GB/s",
                          "tokens_per_s": round(n1 / L * tcheck / s1, 4), "cores": 1},
           "cpu_model": cpu_model(),
           "sample": (f"{layers_done} layer evaluations ({tcheck} token(s) each, replay 0's inputs, every layer "
                      f"at least once) in {secs:.1f}s on {threads} threads; {n1} on one thread in {s1:.1f}s; "
                      f"fp64, OpenMP over output rows; weight generation not timed")}
    return cpu, validated


def rmsnorm_fold_cost(wl, meas, dev):
    """The next layer's RMSNorm on every layer of the step: folded into the tail
    against a separate moe_decode_rmsnorm launch after each layer, each timed
    like the plain step (same n, 5 samples, median) in this process."""
    import torch
    import moe_inputs as mi
    from quantized_moe_decode_amd.layer import tensor_from_encoded
    cfg, L, n = wl.cfg, wl.L, meas["n"]
    weights = [tensor_from_encoded(mi.gen_norm_weight(cfg, li), mi.BF16, dev) for li in range(L)]

    def step_ms():
        wl.step.capture()
        for i in range(max(10, wl.R)):
            wl.step.replay(i % wl.R)
        return statistics.median(timed_replays(wl.step, n, wl.R, offset=k * n) / (n * wl.step.repeat)
                                 for k in range(5)) * 1e3

    plain = step_ms()
    res = {"ms_per_step_plain": round(plain, 4)}
    for fold in (True, False):
        for lay, w in zip(wl.layers, weights):
            lay.set_next_norm(w, cfg.norm_eps, fold=fold)
        ms = step_ms()
        if wl.step.error_words():
            raise SystemExit(f"{cfg.name}: a wait timed out with the RMSNorm")
        key = "folded" if fold else "separate_launch"
        res[f"ms_per_step_{key}"] = round(ms, 4)
        res[f"{key}_us_per_layer"] = round((ms - plain) * 1e3 / L, 3)
    for lay in wl.layers:
        lay.norm_w, lay.normed, lay.tail_ws = None, None, None
    wl.step.capture()
    torch.cuda.synchronize()
    return res


def dtype_of(cfg) -> str:
    w = f"u{cfg.bits_gate_up}" if cfg.bits_gate_up == cfg.bits_down else f"u{cfg.bits_gate_up}/u{cfg.bits_down}"
    acc = f"{cfg.x_dtype} x, f32 accumulation, act staged as f16 (power-of-two scaled) for the down projection"
    return f"{w} weights ({cfg.sb_dtype} scale/bias), {acc}"


def run_workload(name, args, dev, overhead, shared_stacks):
    import torch
    import moe_inputs as mi
    cfg = mi.CONFIGS[name]
    L = args.layers or cfg.n_layers
    stacks = shared_stacks.get(cfg.weight_cfg_id) if cfg.n_tokens > 1 else None
    if stacks is not None and len(stacks) < L:
        stacks = None
    grouped = {"auto": None, "decode": False, "grouped": True}[args.expert_path] if cfg.n_tokens > 1 else None
    repeat = args.steps_per_graph or (32 if L == 1 else 1)
    wl = Workload(cfg, L, args.tokens, dev, stacks=stacks[:L] if stacks else None, grouped=grouped, repeat=repeat)
    shared_stacks[cfg.weight_cfg_id] = wl.stacks
    if args.profile_run:
        # for counter collection: a few plain replays of the step
        for i in range(args.steps):
            wl.step.replay(i % wl.R)
        torch.cuda.synchronize()
        if wl.step.error_words():
            raise SystemExit(f"{name}: a wait inside a launch timed out")
        return {"workload": name, "profiled_steps": args.steps, "layers": L}, wl.stacks
    meas = measure(wl, args, overhead, min_steps=args.steps if name == HEADLINE else 0)
    err = wl.step.error_words()
    if err:
        raise SystemExit(f"{name}: a wait inside a launch timed out during the timed samples")
    mean_bytes = float(np.mean(wl.step_bytes))
    gbps = mean_bytes / meas["median"] / 1e9
    res = {
        "workload": name, "value": round(gbps, 2), "unit": "GB/s",
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(cfg.n_tokens / meas["median"], 2),
        "ms_per_step": round(meas["median"] * 1e3, 4),
        "ms_per_step_min": round(meas["min"] * 1e3, 4), "ms_per_step_max": round(meas["max"] * 1e3, 4),
        "samples": len(meas["samples"]), "steps_per_sample": meas["n"],
        "amortisation_ratio_2n": round(meas["amortisation_ratio_2n"], 4),
        "round_trip_overhead_us": round(overhead * 1e6, 1),
        "expert_bytes_per_step": int(mean_bytes), "other_bytes_per_step": int(wl.other_bytes_per_step()),
        "layers": L, "tokens_per_step": cfg.n_tokens, "distinct_tokens": wl.R, "path": wl.path,
        "expert_ffn": "fused" if wl.T == 1 else ("grouped" if wl.layers[0].grouped else "decode"),
        "steps_per_graph": wl.step.repeat,
        "dtype": dtype_of(cfg),
        "config": {"workload": name, "layers": L, "tokens_per_step": cfg.n_tokens, "d_in": cfg.d_in,
                   "d_ff": cfg.d_ff, "experts": cfg.n_experts, "top_k": cfg.top_k,
                   "bits": [cfg.bits_gate_up, cfg.bits_down], "shared_experts": cfg.n_shared,
                   "d_ff_shared": cfg.d_ff_shared, "distinct_tokens": wl.R, "parallelism": "single GPU"},
    }
    res["roofline"] = roofline_of(wl, meas, args)
    if wl.T == 1:
        res["other_path"] = other_path(wl, args)
    if not args.no_cpu_baseline:
        secs = args.cpu_seconds if name == HEADLINE else args.cpu_seconds / 3
        res["cpu_baseline"], res["validated"] = cpu_leg(wl, args, secs)
    else:
        res["cpu_baseline"], res["validated"] = None, None
    if name in (HEADLINE, "qwen3_30b_a3b_moe_batch32"):
        res["rmsnorm_fold"] = rmsnorm_fold_cost(wl, meas, dev)
    log(f"[bench] {name}: {res['ms_per_step']} ms/step, {res['value']} GB/s, "
        f"{res['tokens_per_s']} tok/s (n={meas['n']}, 2n ratio {res['amortisation_ratio_2n']})")
    keep = wl.stacks
    del wl
    torch.cuda.synchronize()
    return res, keep


def main():
    args = parse()
    sys.path.insert(0, ROOT)
    if args.summarize_counters:
        if args.config == "all":
            raise SystemExit("--summarize-counters needs --config")
        rec = summarize_counters(*args.summarize_counters, args.config, args.copy_mib, args.counters_command)
        with open(counters_path(args.config), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MoE decode layer here runs on a single MI355X "
              "and has no multi-GPU path (the sharding design is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    if args.samples < 10:
        raise SystemExit("--samples must be at least 10")

    sampler = state_sampler(args.profile_run)
    import torch
    import moe_inputs as mi
    import quantized_moe_decode_amd  # noqa: F401  (fails loudly without the built library)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    names = ALL_CONFIGS if args.config == "all" else [args.config]
    for n in names:
        if n not in mi.CONFIGS:
            raise SystemExit(f"unknown workload {n}")
    if args.profile_run and len(names) != 1:
        raise SystemExit("--profile-run needs --config")
    state_before = sampler.sample() if sampler else None
    overhead = round_trip_overhead()
    results, stacks = {}, {}
    for n in names:
        res, keep = run_workload(n, args, dev, overhead, stacks)
        results[n] = res
        # device weights stay only for a later workload that runs on them
        wid = mi.CONFIGS[n].weight_cfg_id
        if not any(mi.CONFIGS[m].weight_cfg_id == wid for m in names[names.index(n) + 1:]):
            stacks.pop(wid, None)
            del keep
            torch.cuda.empty_cache()
    stacks.clear()
    torch.cuda.empty_cache()
    state_after = sampler.sample() if sampler else None
    if sampler:
        sampler.close()

    head = results[HEADLINE] if HEADLINE in results else results[names[0]]
    ceil = None
    if not args.no_ceiling and not args.profile_run:
        ceil = ceiling(dev, head["expert_bytes_per_step"] // head["layers"])

    copy = None
    if args.profile_run:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        copy = {"kernel": "elementwise mul by 1 (torch)", "bytes_read": n * 4, "bytes_written": n * 4,
                "launches": 3}

    if args.profile_run:
        line = {"profile_run": head, "calibration_copy": copy}
        print(json.dumps(line), flush=True)
        return
    bad = [n for n, r in results.items() if r.get("validated") and not r["validated"]["ok"]]
    line = {
        "metric": "expert-weight HBM GB/s (% of ~8 TB/s) and MoE-layer decode tokens/s",
        "value": None if bad else head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["samples"] * head["steps_per_sample"],
        "warmup": args.warmup,
        "warmup_ms": args.warmup_ms,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded generator; random-init weights of the stated shapes)",
        "config": head["config"],
        "tokens_per_s": head["tokens_per_s"],
        "pct_of_hbm_peak": head["pct_of_hbm_peak"],
        "ms_per_step_min": head["ms_per_step_min"], "ms_per_step_max": head["ms_per_step_max"],
        "samples": head["samples"], "steps_per_sample": head["steps_per_sample"],
        "amortisation_ratio_2n": head["amortisation_ratio_2n"],
        "round_trip_overhead_us": head["round_trip_overhead_us"],
        "bytes_per_sample_min": args.bytes_per_sample,
        "expert_bytes_per_step": head["expert_bytes_per_step"],
        "other_bytes_per_step": head["other_bytes_per_step"],
        "path": head["path"],
        "other_path": head.get("other_path"),
        "roofline": head.get("roofline"),
        "cpu_baseline": head.get("cpu_baseline"),
        "validated": head.get("validated"),
        "rmsnorm_fold": head.get("rmsnorm_fold"),
        "ceiling": ceil,
        "gpu_state": {"before": state_before, "after": state_after},
        "configs": {n: r for n, r in results.items() if r is not head},
    }
    print(json.dumps(line), flush=True)
    if bad:
        log(f"[bench] output check FAILED for {bad}: no value reported")
        sys.exit(1)


if __name__ == "__main__":
    main()
