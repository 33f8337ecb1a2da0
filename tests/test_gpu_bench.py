"""The benchmark's JSON line for every named workload, from one short run each
on the GPU: the fields the line promises are there and hold numbers (a line
that breaks only under a GPU would otherwise surface at measurement time)."""
import contextlib
import io
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

WORKLOADS = ["long_8192", "gqa_causal_4096", "gqa_swa_4096", "varlen_grpo_g8", "decode_grpo_32",
             "grpo_64x8"]


@pytest.mark.parametrize("workload", WORKLOADS)
def test_bench_line(workload):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        rc = bench.main(["--workload", workload, "--steps", "2", "--warmup", "1",
                         "--no-cpu-baseline"])
    assert rc == 0
    line = json.loads(out.getvalue().strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "roofline_per_launch", "cpu_baseline"):
        assert key in line, key
    assert line["value"] > 0 and line["ms_per_step"] > 0 and line["n_gpus"] == 1
    assert line["config"]["workload"] == workload
    rl = line["roofline"]
    assert rl["bound"] in ("mfma", "hbm") and 0 < rl["frac"] < 1
    assert rl["achieved"] > 0 and rl["peak"] > 0
    assert line["roofline_per_launch"]
    for x in line["roofline_per_launch"]:
        assert 0 < x["frac"] < 1 and x["avg_launch_ms"] > 0
