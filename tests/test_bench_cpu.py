"""Host-side logic of the benchmark (no GPU): the useful-pair count that
the TFLOP/s figures are built on, against brute-force counting of the
oracle's mask, and the single-GPU guard."""
import numpy as np
import pytest

import bench
import oracle
from workloads import WINDOW_INF, make_inputs


@pytest.mark.parametrize("n", [1, 2, 5, 64, 130])
@pytest.mark.parametrize("w,p", [(0, 0), (3, 0), (0, 4), (16, 4), (128, 16), (WINDOW_INF, 0),
                                 (200, 0), (2, 300)])
def test_visible_pairs_closed_form(n, w, p):
    assert bench.visible_pairs_per_head(n, w, p) == int(oracle.visible_mask(n, w, p).sum())


def test_useful_pairs_varlen_and_batched():
    inp = make_inputs(batch=0, seqlen=0, heads_q=4, heads_kv=2, head_dim=8, window=5, prefix=2,
                      seed=1, dtype="fp32", lengths=(3, 0, 17))
    want = 4 * sum(int(oracle.visible_mask(n, 5, 2).sum()) for n in (3, 0, 17))
    assert bench.useful_pairs(inp) == want
    inp = make_inputs(batch=3, seqlen=20, heads_q=2, heads_kv=1, head_dim=8, window=WINDOW_INF,
                      prefix=0, seed=1, dtype="fp32")
    assert bench.useful_pairs(inp) == 3 * 2 * 20 * 21 // 2


def test_target_workload_flop_count():
    # T=8192 full causal, Hq=64, d=64: 2,147,745,792 visible pairs, 896 FLOP each
    assert 64 * bench.visible_pairs_per_head(8192, WINDOW_INF, 0) == 2_147_745_792
    assert 64 * bench.visible_pairs_per_head(8192, 128, 4) == 69_168_512


def test_multi_gpu_request_refused():
    assert bench.main(["--gpus", "2"]) == 2


def test_kernel_variant_names():
    import bench
    wide = bench.kernel_variants(64, 128)
    narrow = bench.kernel_variants(32, 128)
    heads4 = bench.kernel_variants(32, 128, 8)
    assert wide == {"fwd_ms": "sinkattn_fwd_bf16_d64", "bwd_dkdv_ms": "sinkattn_bwd_dkdv_bf16_d64",
                    "bwd_dq_ms": "sinkattn_bwd_dq_bf16_d64"}
    assert narrow["fwd_ms"] == "sinkattn_fwd_bf16_d64_k32"
    assert heads4["fwd_ms"] == "sinkattn_fwd_bf16_d64_k32h"
    assert bench.kernel_variants(64, 128, 8) == wide
    win = bench.kernel_variants(32, 128, 8, True)
    assert win["bwd_dq_ms"] == "sinkattn_bwd_dq_bf16_d64_win"
    # the resident-tile window dQ kernel: groups of a multiple of 4, at most 6 key tiles
    assert bench.dq_window_kernel(8192, 8, 128, 4) and bench.dq_window_kernel(8192, 4, 128, 16)
    assert not bench.dq_window_kernel(8192, 2, 128, 4)      # group not a multiple of 4
    assert not bench.dq_window_kernel(8192, 8, 160, 4)      # 1 + 5 + 1 = 7 tiles
    assert not bench.dq_window_kernel(8192, 8, 128, 33)     # two prefix tiles
    assert not bench.dq_window_kernel(8192, 8, 1024, 0)     # wide tiles
    for variants in (narrow, heads4, win):
        for ph, name in variants.items():
            assert bench.kernel_base(name) == wide[ph]
            assert bench.kernel_source_sha(name) == bench.kernel_source_sha(wide[ph])


def test_decode_visible_count():
    import bench

    def brute(n, w, p):
        return sum(1 for k in range(n) if k <= n - 1 and (n - 1 - k <= w or k < p))
    for n in range(0, 70):
        for w in (0, 1, 5, 63, 2**31 - 1):
            for p in (0, 1, 4, 64, 100):
                assert bench.decode_visible(n, w, p) == brute(n, w, p)


def test_kernel_bytes_of_the_long_context_layers():
    from workloads import workload_inputs
    inp = workload_inputs("long_8192")[0]
    q = 8192 * 64 * 64
    k = 8192 * 8 * 64
    rows = 8192 * 64
    assert bench.kernel_bytes(inp, "sinkattn_fwd_bf16_d64") == 2 * (2 * q + 2 * k) + 4 * rows
    assert bench.kernel_bytes(inp, "sinkattn_bwd_dq_bf16_d64") == 2 * (4 * q + 2 * k) + 12 * rows
    # dK/dV: Q, dO, K, V in, dK, dV out (bf16), L and D in: 171.97 MB
    assert bench.kernel_bytes(inp, "sinkattn_bwd_dkdv_bf16_d64") == 171966464


def test_compulsory_bytes_target_layer():
    # T=8192, Hq=64, Hkv=8, d=64: Q, K, V in and O out in bf16 plus l in fp32 is 153.1 MB for
    # the forward; the backward reads Q, K, V, dO and L, D and writes dQ, dK, dV
    inp = make_inputs(batch=1, seqlen=8192, heads_q=64, heads_kv=8, head_dim=64, window=128,
                      prefix=4, seed=0, std=0.5, dtype="bf16")
    q = 8192 * 64 * 64
    k = 8192 * 8 * 64
    rows = 8192 * 64
    fwd, bwd = bench.compulsory_bytes(inp)
    assert fwd == 2 * (q + k + k + q) + 4 * rows == 153_092_096
    assert bwd == 2 * (q + k + k + q) + 4 * 2 * rows + 2 * (q + k + k)


def test_committed_sclk_parses_summary(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "sq_counters_wl.md").write_text(
        "| kernel | grid (threads) | time (us, profiled) | clock (GHz) | MFMA busy |\n"
        "|---|---|---|---|---|\n"
        "| kern_a | 100 | 50.0 | 1.95 | 10 % |\n"
        "| kern_a | 200 | 900.5 | 1.81 | 40 % |\n"
        "| kern_b | 100 | 2000.0 | 1.70 | 40 % |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.committed_sclk("kern_a", "wl") == 1.81     # the longest grid of the kernel
    assert bench.committed_sclk("kern_c", "wl") is None
    assert bench.committed_sclk("kern_a", "other") is None


def test_grpo_compulsory_bytes():
    from workloads import make_grpo_inputs
    inp = make_grpo_inputs(lengths=(10, 20, 30, 40), group_size=2, seed=1, beta=0.04)
    assert bench.grpo_bytes(inp) == 100 * (4 + 4 + 4 + 1 + 4) + 4 * 12 + 8
    inp0 = make_grpo_inputs(lengths=(10, 20), group_size=2, seed=1, beta=0.0)
    assert bench.grpo_bytes(inp0) == 30 * 13 + 2 * 12 + 8


def test_committed_traffic_summaries_parse():
    # every committed counter summary names a known source list and carries the
    # fields bench.py reads; when its hash matches the sources, bench.py reports it
    import glob
    import os
    import re
    files = glob.glob(os.path.join(bench.ROOT, "profiles", "*_traffic.md"))
    assert files
    for path in files:
        txt = open(path).read()
        key = re.search(r"^kernel:\s*(\S+)", txt, re.M).group(1)
        assert bench.kernel_base(key) in bench.KERNEL_SOURCES, path
        workload = os.path.basename(path)[len(key) + 1:-len("_traffic.md")]
        sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt).group(1)
        per_layer = re.findall(r"hbm_bytes_per_launch\[layer (\d+)\]:\s*([0-9.eE+]+)", txt)
        if per_layer:   # attention workloads: one value per layer
            for layer, val in per_layer:
                assert float(val) > 0
                got = bench.committed_traffic(key, workload, int(layer))
                assert (got == float(val)) == (sha == bench.kernel_source_sha(key)), path
        else:           # one library call per step (decode, GRPO)
            val = float(re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt).group(1))
            assert val > 0
            got = bench.committed_traffic(key, workload)
            assert (got == val) == (sha == bench.kernel_source_sha(key)), path


def test_scripts_reference_only_defined_names():
    # a name a function reads from module scope must exist there (or be a
    # builtin): the GPU-only branches of these scripts never run on the CPU, so
    # a stray name would otherwise surface only on the GPU machine
    import builtins
    import os
    import symtable
    scripts = ["bench.py", "__graft_entry__.py", "workloads.py", "tests/parity_util.py",
               "sink_aware_masked_sinkattn_amd/binding.py", "sink_aware_masked_sinkattn_amd/build.py"]
    for rel in scripts:
        path = os.path.join(bench.ROOT, rel)
        if not os.path.exists(path):
            continue
        top = symtable.symtable(open(path).read(), rel, "exec")
        defined = set(dir(builtins)) | {s.get_name() for s in top.get_symbols()
                                        if s.is_assigned() or s.is_imported() or s.is_namespace()}
        missing = []

        def walk(t):
            for s in t.get_symbols():
                if s.is_global() and s.is_referenced() and s.get_name() not in defined:
                    missing.append((t.get_name(), s.get_name()))
            for c in t.get_children():
                walk(c)

        for c in top.get_children():
            walk(c)
        assert not missing, (rel, missing)
