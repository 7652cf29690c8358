"""Host-side tools (no GPU): the benchmark's one-GPU contract and the tables
behind the committed profiles."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_several_gpus():
    # the check runs before torch or the library is imported
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_profiling_workload_tables_are_consistent():
    from attention_flash_attn_fwd_amd import profiling as P
    assert len(set(P.WORKLOADS)) == len(P.WORKLOADS)
    assert set(P.KERNEL_OF) == set(P.WORKLOADS) == set(P.SOURCE_OF)
    for wl in P.WORKLOADS:
        src = os.path.join(ROOT, "attention_flash_attn_fwd_amd", "csrc", P.SOURCE_OF[wl])
        assert os.path.exists(src), wl
        # the kernel named for the workload is defined in that source
        name = P.KERNEL_OF[wl].split("<")[0]
        with open(src) as f:
            assert f"void {name}(" in f.read(), (wl, name)


def test_committed_counter_records_are_well_formed():
    from attention_flash_attn_fwd_amd import profiling as P
    with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
        rec = json.load(f)
    cal = rec["_calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    workloads = [k for k in rec if not k.startswith("_")]
    assert workloads and set(workloads) <= set(P.WORKLOADS)
    for wl in workloads:
        r = rec[wl]
        assert r["kernel"] == P.KERNEL_OF[wl] and r["source"] == P.SOURCE_OF[wl], wl
        assert len(r["source_sha256_16"]) == 16
        assert r["kernel_us"] > 0
        assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"], wl
