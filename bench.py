"""Benchmark of the fused online-softmax attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one attn_fwd call over the whole workload (default: B=2, H=16,
N=M=4096, d=128, bf16, causal -- the configuration the throughput target is
stated on) with inputs already resident in HBM.  Prints ONE JSON line on
stdout; progress goes to stderr.

  value      attention-forward TFLOP/s, 4*N*M*d per head (halved for causal)
             over the timed region
  roofline   the attention kernel against the bf16 dense MFMA peak
             (256 CUs x 2.4 GHz x 4096 flop/clk/CU = 2516.6 TFLOP/s); achieved
             = algorithmic flops per launch / the kernel's average launch
             duration, measured with HIP events on the launch stream: the
             timed region's duration / K (one launch of the kernel per step),
             or the mean of per-launch event pairs with --launch-events;
             traffic = HBM bytes per launch from the committed rocprofv3
             counter summary when it was taken on the current kernel source,
             else null
  cpu_baseline  the float64 oracle timed on this host's cores on a bounded,
             evenly spaced sample of the same workload's query rows
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402

PEAKS_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA, MI355X
HBM_PEAK_GBS = 8000.0
# Device code of each attention kernel whose traffic a committed figure may
# record: the figure's stamp (the planning is covered by the kernel name
# each figure records).
BF16_SOURCES = ["attn_bf16.hip", "attn_bf16_common.h"]
KERNEL_SOURCES = {
    "attn_fwd_bf16_w8_kernel": BF16_SOURCES,
    "attn_fwd_bf16_kernel": BF16_SOURCES,
    "attn_fwd_bf16_kh_kernel": BF16_SOURCES,
    "attn_fwd_bf16_kh_bias_kernel": BF16_SOURCES,
    "attn_decode_kernel": ["attn_decode.hip"],
    "attn_fwd_f32_small_kernel": ["attn_f32.hip"],
    "attn_fwd_f32_kernel": ["attn_f32.hip"],
}


def err(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    """Hash of the device sources of `kernel`: // comments, trailing blanks
    and empty lines are dropped, so a comment-only edit keeps the stamp."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "online_softmax_10_amd", "csrc", name), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode("utf-8") + b"\n")
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str, path: str = ""):
    """HBM bytes per launch from the committed counter summary, if it covers this
    kernel and matches the current kernel source."""
    path = path or os.path.join(ROOT, "profiles", f"traffic_attn_fwd_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        t = json.load(f)
    if t.get("kernel") != kernel or t.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


COPY_MIB = 512  # size of the plain copy that calibrates the byte counters


def counter_commands(wl: str, out_dir: str) -> list:
    """The four rocprofv3 counter runs (from the repository root, results
    under out_dir) that --traffic-from-counters reads back."""
    run = f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --trials 0 --no-gemm-ceiling --workload {wl}"
    cal = f"python3 bench.py --calibrate-copy {COPY_MIB} --steps 3"
    pmc = "timeout -s KILL 120 rocprofv3 --pmc"
    return [f"{pmc} FETCH_SIZE --output-format csv -d {out_dir}/pmc_fetch_{wl} -o run -- {run}",
            f"{pmc} WRITE_SIZE --output-format csv -d {out_dir}/pmc_write_{wl} -o run -- {run}",
            f"{pmc} FETCH_SIZE --output-format csv -d {out_dir}/pmc_fetch_copy -o run -- {cal}",
            f"{pmc} WRITE_SIZE --output-format csv -d {out_dir}/pmc_write_copy -o run -- {cal}"]


def traffic_from_counters(wl: str, kernel: str, out_dir: str, dest: str = "") -> dict:
    """HBM bytes per launch of `kernel` from FETCH_SIZE / WRITE_SIZE runs (KiB
    per dispatch, first dispatch dropped), each scaled by what the same counter
    reads for a plain copy of known size; written to
    profiles/traffic_attn_fwd_<wl>.json with the current kernel-source hash."""
    import collections
    import csv
    import glob

    def per_dispatch(sub, match):
        path = glob.glob(os.path.join(out_dir, sub, "**", "*counter_collection.csv"), recursive=True)[0]
        per = collections.defaultdict(float)
        with open(path, newline="", encoding="utf-8") as f:
            for r in csv.DictReader(f):
                if match(r["Kernel_Name"]):
                    per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        return [per[key] for key in sorted(per)]

    is_kernel = lambda name: (kernel + "<") in name
    is_copy = lambda name: "copyBuffer" in name
    fetch = per_dispatch(f"pmc_fetch_{wl}", is_kernel)[1:]
    write = per_dispatch(f"pmc_write_{wl}", is_kernel)[1:]
    cf = per_dispatch("pmc_fetch_copy", is_copy)
    cw = per_dispatch("pmc_write_copy", is_copy)
    if not (fetch and write and cf and cw):
        raise RuntimeError("counter runs hold no dispatches of the expected kernels")
    copy_kib = COPY_MIB * 1024
    ff = copy_kib / (sum(cf) / len(cf))
    fw = copy_kib / (sum(cw) / len(cw))
    fk = sum(fetch) / len(fetch)
    wk = sum(write) / len(write)
    out = {
        "workload": wl,
        "kernel": kernel,
        "kernel_source_hash": kernel_source_hash(kernel),
        "fetch_kib_per_dispatch": round(fk, 1),
        "write_kib_per_dispatch": round(wk, 1),
        "copy_calibration": {"bytes": copy_kib * 1024, "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
        "hbm_bytes_per_launch": round((fk * ff + wk * fw) * 1024),
        "commands": counter_commands(wl, out_dir) + [f"python3 bench.py --workload {wl} --traffic-from-counters {out_dir}"],
        "note": "KiB per dispatch averaged over the timed dispatches (first excluded); factors = copied bytes / "
                "counter bytes for a plain device copy",
    }
    dest = dest or os.path.join(ROOT, "profiles", f"traffic_attn_fwd_{wl}.json")
    with open(dest, "w", encoding="utf-8") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def algorithmic_bytes(w: si.Workload) -> float:
    esz = 2 if w.dtype == "bf16" else 4
    return w.B * w.H * ((w.N + 2 * w.M) * w.d * esz + w.N * w.d * esz + w.N * 4)


def parity_rule(o, lse, o_ref, lse_ref, dtype: str) -> dict:
    """The workloads' element-wise rule, applied to the GPU rows against the oracle's.

    bf16: |o - o_ref| <= 1e-2 + half a bf16 ulp of o_ref (o is stored in bf16)
    and |lse - lse_ref| <= 5e-3; fp32: 1e-5 on both."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    if dtype == "bf16":
        a = np.abs(o_ref)
        half_ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 8.0), 0.0)
        bound, lse_tol = 1e-2 + half_ulp, 5e-3
        rule = "|do| <= 1e-2 + ulp_bf16(o_ref)/2, |dlse| <= 5e-3"
    else:
        bound, lse_tol = np.full_like(o_ref, 1e-5), 1e-5
        rule = "|do| <= 1e-5, |dlse| <= 1e-5"
    err_o = np.abs(o - o_ref)
    err_l = np.abs(np.asarray(lse, dtype=np.float64) - np.asarray(lse_ref, dtype=np.float64))
    ok = bool(np.all(np.isfinite(o)) and np.all(err_o <= bound) and np.all(err_l <= lse_tol))
    return {"rule": rule, "pass": ok, "o_elements_over_bound": int(np.sum(~(err_o <= bound))),
            "lse_over_bound": int(np.sum(~(err_l <= lse_tol))),
            "max_abs_o": float(err_o.max(initial=0.0)), "max_abs_lse": float(err_l.max(initial=0.0))}


def cpu_baseline(w: si.Workload, q, k, v, o_gpu, lse_gpu, target_s: float, bias=None):
    """Time the oracle on an evenly spaced sample of query rows (~target_s seconds)
    and check the GPU's rows of that sample against it (the workloads' rule)."""
    import oracle

    err(f"[bench] cpu baseline: oracle on {oracle.num_threads()} threads")
    qf, kf, vf = (si.to_f64(a, w.dtype) for a in (q, k, v))
    total = w.B * w.H * w.N

    def row_flops(rows):
        i = rows % w.N
        vis = np.minimum(i + 1, w.M) if w.causal else np.full_like(i, w.M)
        return float(np.sum(4.0 * w.d * vis))

    def run(rows):
        t0 = time.perf_counter()
        o, lse = oracle.attention_rows(qf, kf, vf, w.scale, w.causal, rows, bias=bias)
        return time.perf_counter() - t0, o, lse

    probe = np.linspace(0, total - 1, 256).astype(np.int64)
    dt, _, _ = run(probe)
    rate = row_flops(probe) / max(dt, 1e-6)
    count = int(min(total, max(256, 256 * target_s * rate / max(row_flops(probe), 1.0))))
    rows = np.linspace(0, total - 1, count).astype(np.int64)
    dt, o_ref, lse_ref = run(rows)
    flops = row_flops(rows)
    o_s = o_gpu.reshape(-1, w.d)[rows]
    l_s = lse_gpu.reshape(-1)[rows]
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{count} of {total} query rows, evenly spaced over all heads and positions "
                  f"({flops / 1e9:.2f} GFLOP, {dt:.1f} s)",
        "seconds": dt,
        "parity_vs_gpu": dict(parity_rule(o_s, l_s, o_ref, lse_ref, w.dtype), rows_checked=count),
    }


def bench_softmax(args, torch, osa) -> int:
    """online_softmax at bandwidth scale: one read and one write of the matrix per
    step (--softmax-out y), plus the row LSE (y+lse), or the row LSE alone, one
    read of the matrix (lse)."""
    import oracle

    rows, n = (int(t) for t in args.softmax.lower().split("x"))
    x_host = si.make_rows(rows, n, seed=args.seed, spread=4.0)
    x = torch.from_numpy(x_host).cuda()
    mode = args.softmax_out
    y = torch.empty_like(x) if mode != "lse" else None
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda") if mode != "y" else None

    def step():
        if mode == "y":
            osa.online_softmax(x, out=y)
        elif mode == "y+lse":
            osa.online_softmax(x, out=y, return_lse=True, lse=lse)
        else:
            osa.logsumexp(x, out=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))
    # x read once; y written once; 4 bytes per row of LSE.
    nbytes = (rows * n * 4.0) * (1 if mode == "lse" else 2) + (rows * 4.0 if mode != "y" else 0.0)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    # Oracle on evenly spaced rows (bounded), also the parity spot check.
    sample = np.linspace(0, rows - 1, min(rows, max(2048, (1 << 26) // n))).astype(np.int64)
    xs = x_host[sample].astype(np.float64)
    tc = time.perf_counter()
    ref = oracle.softmax(xs) if mode != "lse" else None
    ref_lse = oracle.logsumexp(xs) if mode != "y" else None
    dt = time.perf_counter() - tc
    err_max = {}
    if y is not None:
        err_max["y"] = float(np.max(np.abs(y.cpu().numpy()[sample].astype(np.float64) - ref)))
    if lse is not None:
        err_max["lse"] = float(np.max(np.abs(lse.cpu().numpy()[sample].astype(np.float64) - ref_lse)))
    line = {
        "metric": "online_softmax GB/s at 1 GPU" if mode == "y" else f"online_softmax ({mode}) GB/s at 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"online_softmax rows={rows} n={n} float32, N(0, 4^2) logits, seed {args.seed}, "
                               f"outputs {mode}",
                   "rows": rows, "n": n, "outputs": mode},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": None, "kernel": "online_softmax",
                     "launch_us": round(launch_ms * 1e3, 2), "algorithmic_bytes": nbytes},
        "cpu_baseline": {"value": round(nbytes * len(sample) / rows / dt / 1e9, 3), "unit": "GB/s",
                         "cores": oracle.num_threads(),
                         "kind": "oracle", "sample": f"{len(sample)} of {rows} rows, evenly spaced ({dt:.2f} s)"},
        "max_abs_err_vs_oracle": err_max,
    }
    print(json.dumps(line), flush=True)
    return 0


def time_gemm(torch, n: int, steps: int, warmup: int, seed: int):
    """torch.mm (hipBLASLt) on bf16 n x n matrices of N(0,1) values, timed like
    attention (one timed region of `steps` launches): (ms per launch, TFLOP/s)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    a = torch.randn((n, n), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(warmup):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        torch.mm(a, b, out=c)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del a, b, c
    return ms, 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def bench_gemm(args, torch) -> int:
    """The dense matrix-core rate the chip sustains on random data."""
    n = args.gemm_ceiling
    ms, tflops = time_gemm(torch, n, args.steps, args.warmup, args.seed)
    print(json.dumps({"metric": "bf16 GEMM TFLOP/s (torch.mm, vendor library)", "value": round(tflops, 1),
                      "unit": "TFLOP/s", "n": n, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(ms, 4), "pct_of_bf16_peak": round(100 * tflops / PEAKS_TFLOPS["bf16"], 2),
                      "data": "N(0,1) bf16"}), flush=True)
    return 0


def bench_xent(args, torch, osa) -> int:
    """softmax_xent at bandwidth scale: the logits are read once per step."""
    import oracle

    rows, n = (int(t) for t in args.xent.lower().split("x"))
    x_host = si.make_rows(rows, n, seed=args.seed, spread=4.0)
    lab_host = np.random.default_rng(args.seed + 1).integers(0, n, size=rows).astype(np.int64)
    x = torch.from_numpy(x_host).cuda()
    lab = torch.from_numpy(lab_host).cuda()
    loss = torch.empty((rows,), dtype=torch.float32, device="cuda")
    lse = torch.empty_like(loss)
    for _ in range(args.warmup):
        osa.softmax_xent(x, lab, out=loss, lse=lse)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        _, _, mean = osa.softmax_xent(x, lab, out=loss, lse=lse)
        ends[i].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))
    nbytes = rows * n * 4.0 + rows * (8 + 4 + 4) + 4  # logits once, labels, loss, lse, mean
    sample = np.linspace(0, rows - 1, min(rows, max(512, (1 << 25) // n))).astype(np.int64)
    tc = time.perf_counter()
    ref_loss, ref_lse, _ = oracle.cross_entropy(x_host[sample].astype(np.float64), lab_host[sample])
    dt = time.perf_counter() - tc
    got = loss.cpu().numpy()[sample].astype(np.float64)
    line = {
        "metric": "softmax_xent GB/s at 1 GPU",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"softmax_xent rows={rows} n={n} float32, N(0, 4^2) logits, uniform labels, "
                               f"seed {args.seed}", "rows": rows, "n": n},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (launch_ms * 1e-3) / 1e9, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(nbytes / (launch_ms * 1e-3) / 1e9 / 8000.0, 4), "traffic": None,
                     "kernel": "softmax_xent_kernel + xent_mean_kernel", "launch_us": round(launch_ms * 1e3, 2),
                     "algorithmic_bytes": nbytes},
        "cpu_baseline": {"value": round(len(sample) * n * 4.0 / dt / 1e9, 3), "unit": "GB/s",
                         "cores": oracle.num_threads(), "kind": "oracle",
                         "sample": f"{len(sample)} of {rows} rows, evenly spaced ({dt:.2f} s)"},
        "max_abs_err_vs_oracle": {"loss": float(np.max(np.abs(got - ref_loss)))},
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # Untimed steps before the timed region.  The chip's clock ramps up over
    # the first tens of milliseconds of sustained matrix-core load: on the
    # 2x16x4096^2 causal workload the timed region read 153 us per step
    # after 5 warm-up steps, 132 after 100 and 127 after 300 (one box).
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="c3", choices=sorted(si.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch-events", action="store_true",
                    help="also record an event pair around every step (adds a GPU drain per step)")
    ap.add_argument("--order", default="q_outer", choices=["q_outer", "kv_outer"],
                    help="loop order of the attention: the fused query-outer kernels (default) or the "
                         "key/value-outer order with the row state through HBM (attn_fwd_kv_outer)")
    ap.add_argument("--bias", action="store_true",
                    help="attention with an additive [N,M] float32 score bias broadcast over batch and heads")
    ap.add_argument("--softmax", default="", metavar="ROWSxN",
                    help="instead of attention, time the row-wise online_softmax on a ROWS x N float32 matrix "
                         "(e.g. 32768x1024: the rows and key count of the 4x8x1024 workload)")
    ap.add_argument("--softmax-out", default="y", choices=["y", "y+lse", "lse"],
                    help="with --softmax: the outputs written (softmax rows, rows and their LSE, or the LSE alone)")
    ap.add_argument("--xent", default="", metavar="ROWSxN",
                    help="instead of attention, time softmax_xent (per-row cross-entropy + mean) on ROWS x N "
                         "float32 logits (e.g. 8192x32000)")
    ap.add_argument("--trials", type=int, default=5,
                    help="further timed regions of K steps each after the main one, reported as their median")
    ap.add_argument("--gemm-ceiling", type=int, default=0, metavar="N",
                    help="only time torch.mm on N x N bf16 matrices of N(0,1) values (the vendor GEMM): the "
                         "matrix-core rate this chip sustains on random data, for comparison with attention")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps in one HIP graph and replay it (the trials replay it again): "
                         "the device's rate for launches shorter than the host's per-call work")
    ap.add_argument("--no-gemm-ceiling", action="store_true",
                    help="skip the vendor bf16 GEMM timed after a bf16 attention run (bf16_gemm_ceiling)")
    ap.add_argument("--copy-rate", type=int, default=0, metavar="MIB",
                    help="only time torch's device copy of MIB MiB (read + write GB/s): the rate a plain copy reaches")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--traffic-from-counters", default="", metavar="DIR",
                    help="no GPU work: read the FETCH_SIZE / WRITE_SIZE counter runs of --workload and of the "
                         "copy calibration under DIR and write profiles/traffic_attn_fwd_<workload>.json")
    args = ap.parse_args()
    if args.traffic_from_counters:
        import online_softmax_10_amd as osa

        w = si.WORKLOADS[args.workload]
        kernel = osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype)[0]
        print(json.dumps(traffic_from_counters(args.workload, kernel, args.traffic_from_counters), indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        return 2

    import torch

    import online_softmax_10_amd as osa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 4 * n, "launches": args.steps}), flush=True)
        return 0
    if args.copy_rate:
        # torch's device-to-device copy (the vendor's streaming kernel), timed
        # like the kernels here: the HBM rate a plain copy reaches.
        n = args.copy_rate * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        gbs = 2.0 * 4 * n / (ms * 1e-3) / 1e9
        print(json.dumps({"metric": "device copy GB/s (torch copy_, read + write)", "value": round(gbs, 1),
                          "unit": "GB/s", "bytes_read": 4 * n, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": round(ms, 4), "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}),
              flush=True)
        return 0
    if args.gemm_ceiling:
        return bench_gemm(args, torch)
    if args.softmax:
        return bench_softmax(args, torch, osa)
    if args.xent:
        return bench_xent(args, torch, osa)
    if args.graph and (args.order == "kv_outer" or args.launch_events or args.bias):
        print("--graph times the single-launch attention plans only (no --order kv_outer, --launch-events or --bias).",
              file=sys.stderr)
        return 2
    if args.bias and args.order == "kv_outer":
        print("--bias applies to the fused (query-outer) kernels only.", file=sys.stderr)
        return 2
    w = si.WORKLOADS[args.workload]
    err(f"[bench] workload {w}")
    q, k, v = si.make_qkv(w, args.seed)

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    qd, kd, vd = dev(q), dev(k), dev(v)
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=tdtype, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    bias_host = bias_dev = None
    if args.bias:
        # [N, M] float32 bias broadcast over batch and heads.
        bias_host = si.make_bias((w.N, w.M), args.seed + 100)
        bias_dev = torch.from_numpy(bias_host).cuda()
    if args.order == "kv_outer":
        def step():
            osa.fwd_kv_outer(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse)
    elif args.bias:
        def step():
            osa.fwd(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse, bias=bias_dev)
    else:
        def step():
            osa.fwd(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region holds exactly K steps between two events on the launch
    # stream.  Per-launch events (--launch-events) make the GPU drain and write
    # a timestamp between kernels, which costs a few microseconds per step,
    # so by default the kernel's average launch duration is the region's
    # duration / K (each step is one launch of the dominant kernel; any gap
    # between launches is counted, so it is an upper bound).
    stream = torch.cuda.current_stream()
    run_steps = None
    if args.graph and osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype)[1] != 1:
        print("--graph times the single-launch attention plans only (this workload splits its keys).", file=sys.stderr)
        return 2
    if args.graph:
        # The K steps captured once in a HIP graph and replayed: the launches
        # go out without the host's per-call work in between (for problems
        # whose launch is shorter than the binding's call).
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(args.steps):
                    step()
        stream.wait_stream(side)
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()
        run_steps = graph.replay
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] if args.launch_events else []
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] if args.launch_events else []
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    if run_steps is not None:
        run_steps()
    else:
        for i in range(args.steps):
            if args.launch_events:
                starts[i].record(stream)
            step()
            if args.launch_events:
                ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = t_begin.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # Five further timed regions of K steps each: the spread between them
    # (the clock falls under sustained matrix-core load) beside the main one.
    trial_us = []
    if args.trials > 0:
        ta, tb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.trials):
            torch.cuda.synchronize()
            ta.record(stream)
            if run_steps is not None:
                run_steps()
            else:
                for _ in range(args.steps):
                    step()
            tb.record(stream)
            torch.cuda.synchronize()
            trial_us.append(ta.elapsed_time(tb) / args.steps * 1e3)
    if args.launch_events:
        launch_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))
    else:
        launch_ms = ms_per_step
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    err(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (host wall {wall / args.steps * 1e6:.1f} us), "
        f"{value:.1f} TFLOP/s")

    kernel, splits = osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype)
    if args.order == "kv_outer":
        kernel, splits = "attn_kv_block_kernel (one launch per 64-key block)", 1
    abytes = algorithmic_bytes(w)
    if args.bias:
        # Bias calls take the bias instantiation of the width the plan names
        # (never the decode kernel).
        if w.dtype != "bf16":
            kernel = "attn_fwd_f32_kernel"
        else:
            kernel = {"attn_fwd_bf16_w8_kernel": "attn_fwd_bf16_w8_bias_kernel",
                      "attn_fwd_bf16_kh_kernel": "attn_fwd_bf16_kh_bias_kernel" if w.d == 64
                      else "attn_fwd_bf16_bias_kernel"}.get(kernel, "attn_fwd_bf16_bias_kernel")
        abytes += w.N * w.M * 4  # the broadcast bias, read once
    achieved = w.flops / (launch_ms * 1e-3) / 1e12
    gbs = abytes / (launch_ms * 1e-3) / 1e9
    # The decode kernel reads each key and value once for a handful of
    # queries: bound by HBM, not by the matrix cores.
    hbm_bound = kernel == "attn_decode_kernel"
    peak = HBM_PEAK_GBS if hbm_bound else PEAKS_TFLOPS[w.dtype]
    roofline = {
        "bound": "hbm" if hbm_bound else "mfma",
        "achieved": round(gbs if hbm_bound else achieved, 2),
        "peak": peak,
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "frac": round((gbs if hbm_bound else achieved) / peak, 4),
        # HBM bytes per launch of the kernel named, from the committed
        # counter runs (a split call also runs the small merge kernel).
        "traffic": load_traffic(w.name, kernel) if (splits == 1 or hbm_bound) and not args.bias else None,
        "kernel": kernel,
        "splits": splits,
        "launch_us": round(launch_ms * 1e3, 2),
        "launch_timing": ("per-launch event pairs" if args.launch_events else
                          "timed region / steps" + (", the steps replayed from one HIP graph" if args.graph else "")),
        "achieved_from": ("algorithmic work of one call / launch_us" +
                          ("" if args.launch_events else
                           ", launch_us = the timed region / steps: the gaps between launches count against "
                           "the kernel (the rocprofv3 kernel trace gives the kernel alone)")),
        "algorithmic_bytes": abytes,
        "hbm_gbs_algorithmic": round(gbs, 1),
    }
    if hbm_bound:
        roofline["tflops"] = round(achieved, 2)

    # The vendor bf16 GEMM on random data in the same process, after the
    # attention timing: the matrix-core rate this chip sustains, beside the
    # share of the published peak.
    gemm_ceiling = None
    if w.dtype == "bf16" and not args.no_gemm_ceiling and args.order == "q_outer" and not hbm_bound:
        gms, gtf = time_gemm(torch, 8192, 20, 50, args.seed)
        gemm_ceiling = {"what": "torch.mm bf16 8192^3, N(0,1) operands (hipBLASLt), 20 launches after 50",
                        "tflops": round(gtf, 1), "pct_of_bf16_peak": round(100.0 * gtf / PEAKS_TFLOPS["bf16"], 2),
                        "value_over_ceiling": round(value / gtf, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        o_host = o.float().cpu().numpy().astype(np.float64)
        l_host = lse.cpu().numpy().astype(np.float64)
        cpu = cpu_baseline(w, q, k, v, o_host, l_host, args.cpu_seconds,
                           None if bias_host is None else bias_host.astype(np.float64))

    line = {
        "metric": "attn fwd TFLOP/s at 1 GPU + % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} "
                               f"{'causal' if w.causal else 'non-causal'}, seed {args.seed}"
                               + (", key/value-outer loop order" if args.order == "kv_outer" else "")
                               + (", additive [N,M] fp32 bias N(0, 2^2) broadcast over batch and heads"
                                  if args.bias else ""),
                   "B": w.B, "H": w.H, "N": w.N, "M": w.M, "d": w.d, "causal": w.causal},
        "pct_of_bf16_peak": round(100.0 * value / PEAKS_TFLOPS["bf16"], 2),
        "bf16_gemm_ceiling": gemm_ceiling,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if trial_us:
        line["trials"] = {"count": len(trial_us), "steps_each": args.steps,
                          "us_per_step": [round(t, 2) for t in trial_us],
                          "median_us_per_step": round(float(np.median(trial_us)), 2),
                          "median_tflops": round(w.flops / (float(np.median(trial_us)) * 1e-6) / 1e12, 2),
                          "note": "run after the main timed region, which alone gives value"}
    print(json.dumps(line), flush=True)
    if cpu is not None and not cpu["parity_vs_gpu"]["pass"]:
        err(f"[bench] the GPU output fails the parity rule against the oracle: {cpu['parity_vs_gpu']}")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
