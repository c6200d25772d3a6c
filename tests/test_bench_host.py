"""Host logic of bench.py (CPU only): the workload's algorithmic flops and
bytes, the one-GPU refusal, the counter -> HBM-bytes arithmetic and the
kernel-source stamp that retires a stale traffic figure."""

import json
import os
import subprocess
import sys

import pytest

import bench
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_of_the_bench_workload():
    w = si.WORKLOADS["c3"]
    # 4 N M d per head, halved for the causal mask: 2*16 heads.
    assert w.flops == 0.5 * 4 * 32 * 4096 * 4096 * 128 == 137438953472.0
    # Q, K, V read once (bf16), O written once (bf16), LSE written once (fp32).
    per_head = 3 * 4096 * 128 * 2 + 4096 * 128 * 2 + 4096 * 4
    assert bench.algorithmic_bytes(w) == 32 * per_head == 134742016
    c1 = si.WORKLOADS["c1"]  # fp32, non-causal
    assert c1.flops == 4 * 256 * 256 * 64
    assert bench.algorithmic_bytes(c1) == (3 * 256 * 64 + 256 * 64) * 4 + 256 * 4


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", encoding="utf-8") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for d, name, v in rows:
            f.write(f'{d},"{name}",C,{v}\n')


def test_traffic_from_counters(tmp_path):
    k = "attn_fwd_bf16_w8_kernel"
    kname = f"void osa::(anonymous namespace)::{k}<128, true, false>(unsigned short const*)"
    copy = "__amd_rocclr_copyBuffer"
    # Three dispatches per run; the first (warm-up) is dropped.  Counter
    # values are summed over the rows of one dispatch (one row per XCD).
    _counter_csv(str(tmp_path / "pmc_fetch_c3" / "run_counter_collection.csv"),
                 [(1, kname, 999.0), (2, kname, 60.0), (2, kname, 40.0), (3, kname, 100.0)])
    _counter_csv(str(tmp_path / "pmc_write_c3" / "run_counter_collection.csv"),
                 [(1, kname, 7.0), (2, kname, 50.0), (3, kname, 50.0)])
    # Copy calibration: FETCH reads half the copied KiB, WRITE all of it.
    half, full = 512 * 1024 / 2, 512 * 1024
    _counter_csv(str(tmp_path / "pmc_fetch_copy" / "run_counter_collection.csv"), [(1, copy, half), (2, copy, half)])
    _counter_csv(str(tmp_path / "pmc_write_copy" / "run_counter_collection.csv"), [(1, copy, full), (2, copy, full)])
    dest = str(tmp_path / "traffic.json")
    t = bench.traffic_from_counters("c3", k, str(tmp_path), dest)
    assert t["copy_calibration"]["fetch_factor"] == 2.0 and t["copy_calibration"]["write_factor"] == 1.0
    assert t["fetch_kib_per_dispatch"] == 100.0 and t["write_kib_per_dispatch"] == 50.0
    assert t["hbm_bytes_per_launch"] == (100 * 2 + 50 * 1) * 1024
    with open(dest, encoding="utf-8") as f:
        assert json.load(f)["kernel_source_hash"] == bench.kernel_source_hash(k)
    # Read back only for the same kernel and the same kernel sources.
    assert bench.load_traffic("c3", k, dest) == t["hbm_bytes_per_launch"]
    assert bench.load_traffic("c3", "attn_fwd_bf16_kernel", dest) is None
    stale = dict(t, kernel_source_hash="0" * 16)
    with open(dest, "w", encoding="utf-8") as f:
        json.dump(stale, f)
    assert bench.load_traffic("c3", k, dest) is None


def test_source_stamp_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "online_softmax_10_amd" / "csrc"
    src.mkdir(parents=True)
    names = sorted({n for srcs in bench.KERNEL_SOURCES.values() for n in srcs})
    for name in names:
        (src / name).write_text("int a = 1;  // one\n\n// note\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    k = "attn_fwd_bf16_w8_kernel"
    h0 = {kern: bench.kernel_source_hash(kern) for kern in bench.KERNEL_SOURCES}
    first = bench.KERNEL_SOURCES[k][0]
    (src / first).write_text("int a = 1;  // another note\n// more\nint b = 2;   \n")
    assert bench.kernel_source_hash(k) == h0[k]
    (src / first).write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash(k) != h0[k]
    # a kernel whose sources did not change keeps its stamp
    assert bench.kernel_source_hash("attn_decode_kernel") == h0["attn_decode_kernel"]


def test_committed_traffic_matches_the_sources():
    # The committed counter summaries were taken on the current kernels.
    for wl in ("c3", "c4", "c5"):
        path = os.path.join(ROOT, "profiles", f"traffic_attn_fwd_{wl}.json")
        with open(path, encoding="utf-8") as f:
            t = json.load(f)
        if t["kernel_source_hash"] != bench.kernel_source_hash(t["kernel"]):
            pytest.fail(f"{path} was taken on other kernel sources; re-take the counter runs it lists")
        assert t["hbm_bytes_per_launch"] >= bench.algorithmic_bytes(si.WORKLOADS[wl])
