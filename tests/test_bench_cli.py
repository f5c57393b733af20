"""CPU tests of bench.py's host logic: the one-GPU refusal and the counter
summary (FETCH_SIZE / WRITE_SIZE scaled by a copy kernel of known size)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_counter_summary_scales_by_the_copy_kernel(tmp_path):
    # the layer kernel reads 1000 and writes 100 "raw" units; the 256 MiB copy
    # reads 2 * 256 Mi-KiB raw (a counter that reads twice the bytes) and writes 1x
    k = "void moe::layer_kernel<4, 4, 2, 2, 3>(moe::LayerArgs)"
    c = "void at::native::vectorized_elementwise_kernel<4, MulFunctor<float> >"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _pmc_csv(fetch, "FETCH_SIZE", [(k, 1000), (k, 1000), (c, 2 * 256 * 1024), ("other", 5)])
    _pmc_csv(write, "WRITE_SIZE", [(k, 100), (k, 100), (c, 256 * 1024)])
    rec = bench.summarize_counters(str(fetch), str(write), "qwen3_30b_a3b_moe", 256, "cmd")
    assert rec["kernel"] == bench.FUSED_KERNEL
    assert rec["fetch_scale"] == 0.5 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (1000 * 0.5 + 100) * 1024
    assert rec["launches"] == [2, 2]
    assert rec["sources_sha256"] == bench.kernel_sources_sha256()
    json.dumps(rec)


def test_batch_workload_counts_its_gate_up_kernel():
    import moe_inputs as mi
    assert bench.dominant_kernel(mi.CONFIGS["qwen3_30b_a3b_moe_batch32"]) == bench.BATCH_GATE_UP_KERNEL
    assert bench.dominant_kernel(mi.CONFIGS["qwen3_30b_a3b_moe"]) == bench.FUSED_KERNEL
    assert bench.dominant_kernel(mi.CONFIGS["qwen3_30b_a3b_moe_prefill256"]) == bench.GROUPED_FFN_KERNEL


def test_prefill_workload_reuses_the_headline_weights_and_takes_the_grouped_path():
    import moe_inputs as mi
    import quantized_moe_decode_amd as qmd
    p, h = mi.CONFIGS["qwen3_30b_a3b_moe_prefill256"], mi.CONFIGS["qwen3_30b_a3b_moe"]
    assert p.weight_cfg_id == h.weight_cfg_id and p.cfg_id != h.cfg_id
    assert qmd.MOE_MAX_TOKENS < p.n_tokens <= qmd.MOE_MAX_GROUPED_TOKENS
    assert bench.MAX_DECODE_TOKENS == qmd.MOE_MAX_TOKENS
    assert bench.ALL_CONFIGS.index("qwen3_30b_a3b_moe_prefill256") == 2


def test_counter_summary_of_the_grouped_unit_sums_its_kernels(tmp_path):
    """On the grouped path the roofline unit is one grouped expert FFN call:
    bucketing + the gate/up-and-down launch, per-dispatch means summed."""
    b = "moe::grouped_bucket_kernel(int const*, int, int, int, int*, int*, int*, int*, int*, int*, int*, int)"
    f = "void moe::ffn_grouped_fused<2, 2>(moe::GroupedArgs)"
    c = "void at::native::vectorized_elementwise_kernel<4, MulFunctor<float> >"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _pmc_csv(fetch, "FETCH_SIZE", [(b, 1), (b, 3), (f, 1500), (f, 1500), (c, 256 * 1024),
                                   ("void moe::route_logits_mfma(moe::RouteArgs)", 77)])
    _pmc_csv(write, "WRITE_SIZE", [(b, 0), (b, 0), (f, 300), (f, 300), (c, 256 * 1024)])
    rec = bench.summarize_counters(str(fetch), str(write), "qwen3_30b_a3b_moe_prefill256", 256, "cmd")
    assert rec["kernel"] == " + ".join([bench.GROUPED_BUCKET_KERNEL, bench.GROUPED_FFN_KERNEL])
    assert rec["hbm_bytes_per_launch"] == (2 + 1500 + 300) * 1024
    assert rec["launches"] == [2, 2]


def test_a_profile_run_starts_no_helper_process(monkeypatch):
    def refuse():
        raise AssertionError("a profile run started the amd-smi helper")
    monkeypatch.setattr(bench, "GpuStateSampler", refuse)
    assert bench.state_sampler(True) is None
