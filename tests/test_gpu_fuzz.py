"""Seeded random problems against the float64 oracle: batch, heads, query and
key counts, head size, dtype, causal alignment, key lengths, an additive bias
(full or broadcast) and the split count drawn independently per case, so
combinations no hand-written case covers still meet the tolerance rule."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import compare, f32_bounds, log, to_device

pytestmark = pytest.mark.gpu

CASES = 48


def draw(case: int):
    rng = np.random.default_rng(9000 + case)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    N = int(rng.choice([int(rng.integers(1, 6)), int(rng.integers(1, 300)), int(rng.integers(300, 700))]))
    M = int(rng.choice([int(rng.integers(1, 70)), int(rng.integers(64, 400)), int(rng.integers(400, 1100))]))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    causal = [False, True, "bottom_right"][int(rng.integers(0, 3))]
    kv_len = [int(x) for x in rng.integers(0, M + 1, size=B)] if rng.random() < 0.4 else None
    bias = None
    r = rng.random()
    if r < 0.2:
        bias = (B, H, N, M)
    elif r < 0.35:
        bias = (N, M)
    elif r < 0.45:
        bias = (1, H, 1, M)
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    dist = ["normal", "uniform01", "normal_qk3"][int(rng.integers(0, 3))]
    return si.Workload("fuzz", B, H, N, M, d, dtype, causal is not False, dist), causal, kv_len, bias, splits


@pytest.mark.parametrize("case", range(CASES))
def test_random_problem(case):
    import torch

    import online_softmax_10_amd as osa

    w, causal, kv_len, bshape, splits = draw(case)
    log(f"[gpu] fuzz {case}: B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} {w.dist} causal={causal} "
        f"kv_len={kv_len} bias={bshape} splits={splits}")
    q, k, v = si.make_qkv(w, case)
    bias = None if bshape is None else si.make_bias(bshape, case + 500, "normal", 0.05)
    qd, kd, vd = (to_device(a, w.dtype) for a in (q, k, v))
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    o, lse = osa.fwd_splits(qd, kd, vd, scale=w.scale, causal=causal, num_splits=splits, kv_len=kl, bias=bd)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype), w.scale,
                                      causal, kv_len=kv_len, bias=None if bias is None else bias.astype(np.float64))
    vis = np.isfinite(lse_ref)
    assert np.all(o[~vis] == 0.0) and np.all(np.isneginf(lse[~vis])), "rows with no finite score"
    if vis.any():
        bounds = None
        if w.dtype == "f32":
            bo, bl = f32_bounds(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype), w.scale, causal,
                                kv_len=kv_len, bias=None if bias is None else bias.astype(np.float64))
            bounds = (bo[vis], bl[vis])
        compare(o[vis], lse[vis], o_ref[vis], lse_ref[vis], w.dtype, f"fuzz {case}", bounds)


@pytest.mark.parametrize("N,M,causal,dtype", [(1, 300001, False, "bf16"), (5, 262147, "bottom_right", "bf16"),
                                              (130, 200003, False, "bf16"), (3, 100003, "bottom_right", "f32")])
def test_long_key_range(N, M, causal, dtype):
    # Key ranges long enough for the split planner's upper end and long sums.
    import torch

    import online_softmax_10_amd as osa

    w = si.Workload("long", 1, 2, N, M, 128, dtype, causal is not False, "normal")
    log(f"[gpu] long keys N={N} M={M} causal={causal} {dtype} plan={osa.plan(1, 2, N, M, 128, dtype)}")
    q, k, v = si.make_qkv(w, 77)
    qd, kd, vd = (to_device(a, dtype) for a in (q, k, v))
    o, lse = osa.fwd(qd, kd, vd, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), w.scale, causal)
    bounds = None
    if dtype == "f32":
        bounds = f32_bounds(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), w.scale, causal)
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, dtype,
            f"long keys M={M}", bounds)


KH_CASES = 24


def draw_key_halves(case):
    # Problems the key-halves kernel takes: few 128-row query tiles, at least
    # 12 (d = 64) or 16 (d = 128) key tiles; masks, key lengths, a bias at
    # d = 64, the float32 output.
    rng = np.random.default_rng(70000 + case)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    N = int(rng.choice([int(rng.integers(5, 40)), int(rng.integers(40, 700))]))  # above the decode shape
    d = int(rng.choice([64, 128]))
    M = int(rng.integers(12 * 64 + 1 if d == 64 else 15 * 64 + 1, 2500))
    causal = [False, True, "bottom_right"][int(rng.integers(0, 3))]
    kv_len = [int(x) for x in rng.integers(0, M + 1, size=B)] if rng.random() < 0.35 else None
    bias = (N, M) if d == 64 and rng.random() < 0.3 else None
    out_f32 = bias is None and rng.random() < 0.2
    dist = ["normal", "uniform01", "normal_qk3"][int(rng.integers(0, 3))]
    return si.Workload("khfuzz", B, H, N, M, d, "bf16", causal is not False, dist), causal, kv_len, bias, out_f32


@pytest.mark.parametrize("case", range(KH_CASES))
def test_random_key_halves_problem(case):
    import torch

    import online_softmax_10_amd as osa

    w, causal, kv_len, bshape, out_f32 = draw_key_halves(case)
    plan = osa.plan(w.B, w.H, w.N, w.M, w.d, "bf16_out_f32" if out_f32 else "bf16")
    log(f"[gpu] key-halves fuzz {case}: B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dist} causal={causal} "
        f"kv_len={kv_len} bias={bshape} out_f32={out_f32} plan={plan}")
    assert plan == ("attn_fwd_bf16_kh_kernel", 1)
    q, k, v = si.make_qkv(w, 900 + case)
    bias = None if bshape is None else si.make_bias(bshape, case + 1500, "normal", 0.05)
    qd, kd, vd = (to_device(a, "bf16") for a in (q, k, v))
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    o, lse = osa.fwd_splits(qd, kd, vd, scale=w.scale, causal=causal, num_splits=0, kv_len=kl, bias=bd,
                            out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention(si.to_f64(q, "bf16"), si.to_f64(k, "bf16"), si.to_f64(v, "bf16"), w.scale,
                                      causal, kv_len=kv_len, bias=None if bias is None else bias.astype(np.float64))
    vis = np.isfinite(lse_ref)
    assert np.all(o[~vis] == 0.0) and np.all(np.isneginf(lse[~vis])), "rows with no finite score"
    if vis.any():
        compare(o[vis], lse[vis], o_ref[vis], lse_ref[vis], "bf16", f"key-halves fuzz {case}")
