"""bench.py on the CPU: the one-GPU contract and the committed counter files.

The timed run itself needs the GPU; these checks do not."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_hashes_cover_existing_sources():
    for kernel in bench.KERNEL_SOURCES:
        h = bench.source_hash(kernel)
        assert len(h) == 16 and int(h, 16) >= 0


def test_comment_edits_do_not_change_the_hash():
    src = "int f(int x) { return x + 1; } // one\n/* two */\n"
    assert bench._code_only(src) == bench._code_only("int f(int x) {\n  return x + 1;\n}\n")


def test_committed_traffic_files_are_well_formed():
    for name in ("attn_fwd_720p_traffic.json", "attn_qk_prep_720p_traffic.json"):
        d = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert d["bytes_per_launch"] == d["fetch_bytes"] + d["write_bytes"]
        assert d["bytes_per_launch"] >= d["algorithmic_bytes"] * 0.99
        assert 1.9 < d["fetch_scale"] < 2.1 and d["write_scale"] == 1.0
        assert "rocprofv3 --pmc FETCH_SIZE" in d["command_fetch"]
        assert "rocprofv3 --pmc WRITE_SIZE" in d["command_write"]


def test_kernel_short_names():
    from block_sparse_video_frame_amd.profiling import short_name
    ns = "void bsvf::(anonymous namespace)::"
    assert short_name(ns + "fwd_persistent<128, 1, 8, false, true>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[persistent]"
    assert short_name(ns + "fwd_persistent<64, 1, 8, true, true>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[persistent,masked]"
    assert short_name(ns + "fwd_persistent<128, 1, 8, false, false>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[persistent,online]"
    assert short_name(ns + "fwd_persistent<128, 1, 8, false, true, false>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[persistent]"
    assert short_name(ns + "fwd_persistent<128, 1, 8, false, false, false>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[persistent,online]"
    assert short_name(ns + "fwd_persistent<64, 1, 8, false, true, true>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[persistent,checked]"
    assert short_name(ns + "fwd_kernel<128, 1, 8, false, false, true>(bsvf::(anonymous namespace)::FwdArgs)") \
        == "attn_fwd[online,checked]"
    assert short_name(ns + "fwd_kernel<128, 1, 8, true, false>(bsvf::(anonymous namespace)::FwdArgs, int const*)") \
        == "attn_fwd[bound]"
    assert short_name(ns + "fwd_kernel<64, 1, 8, false, true>(bsvf::(anonymous namespace)::FwdArgs, int const*)") \
        == "attn_fwd[online,masked]"
    assert short_name(ns + "head_max_kernel<true>(float const*, float const*, int, float*)") == "attn_norms[head_max]"


def test_cpu_baseline_pool_on_the_tiny_workload():
    """The CPU baseline runs the oracle in a pool of one worker per host core
    over (head, 512-row) tasks and reports the workers as its cores."""
    from synth import WORKLOADS, make_qkv
    wl = WORKLOADS["tiny"]
    q, k, v = make_qkv(wl)
    r = bench.cpu_baseline(wl, q, k, v, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] == r["workers"] == r["host_cores"] == len(os.sched_getaffinity(0))
    assert f"{wl.seq_len} rows" in r["sample"]   # a task holds min(512, N) rows
