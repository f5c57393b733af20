"""The committed profiler summaries: each names the command that produced it,
that command runs only files of this repository, and the counter records are
well-formed.  CPU only."""
import glob
import json
import os
import re

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _md_files():
    files = sorted(glob.glob(os.path.join(PROFILES, "*.md")))
    assert files, "no profiler summaries committed"
    return files


def test_every_summary_gives_its_profiler_command():
    for path in _md_files():
        text = open(path).read()
        blocks = re.findall(r"```\n(.*?)```", text, flags=re.S)
        cmds = [ln for b in blocks for ln in b.splitlines() if "rocprofv3" in ln]
        assert cmds, f"{os.path.basename(path)}: no rocprofv3 command"
        for ln in cmds:
            # the profiled program comes straight after `--` (no launcher in between)
            prog = ln.split(" -- ", 1)[1].split()
            assert prog[0] == "python3", ln
            assert prog[1].startswith("<repo>/"), ln


def test_commands_run_committed_files_only():
    for path in _md_files():
        for rel in re.findall(r"<repo>/([A-Za-z0-9_./]+)", open(path).read()):
            assert not rel.startswith("_work"), (path, rel)
            assert os.path.isfile(os.path.join(ROOT, rel)), (path, rel)


def test_summaries_are_short_text():
    for path in glob.glob(os.path.join(PROFILES, "*")):
        assert path.endswith((".md", ".json")), path
        assert os.path.getsize(path) < 16 * 1024, path


def test_counter_records_are_complete():
    recs = sorted(glob.glob(os.path.join(PROFILES, "counters_*.json")))
    assert recs
    for path in recs:
        r = json.load(open(path))
        assert os.path.basename(path) == f"counters_{r['workload']}.json"
        assert r["workload"] in mi.CONFIGS
        assert re.fullmatch(r"[0-9a-f]{64}", r["sources_sha256"])
        assert min(r["launches"]) > 0 and r["hbm_bytes_per_launch"] > 0   # launches: [fetch run, write run]
        # FETCH_SIZE of the calibration copy reads about half its bytes raw
        # (factor ~2), WRITE_SIZE all of them (factor ~1)
        assert 1.5 < r["fetch_scale"] < 2.5 and 0.8 < r["write_scale"] < 1.25
        assert "rocprofv3" in r["command"] and "<repo>/bench.py" in r["command"]
