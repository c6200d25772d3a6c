"""GPU parity of attn_fwd_masked (through the C ABI) against the float64 oracle:
bottom-right causal masks for N < M and N > M, per-batch key lengths
(including 0 and M), their combinations, on every kernel path (bf16 four- and
eight-wave, fp32, decode, forced splits).  Rows with no visible key must come
back as o = 0, lse = -inf."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import compare, f32_bounds, log, to_device

pytestmark = pytest.mark.gpu


def run_masked(w, causal, kv_len, splits=0, seed=0):
    import torch

    import online_softmax_10_amd as osa

    q, k, v = si.make_qkv(w, seed)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    log(f"[gpu] masked B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} causal={causal} kv_len={kv_len} "
        f"splits={splits} kernel={osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype, splits)}")
    qd, kd, vd = (to_device(a, w.dtype) for a in (q, k, v))
    o, lse = osa.fwd_splits(qd, kd, vd, scale=w.scale, causal=causal, num_splits=splits, kv_len=kl)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype),
                                      w.scale, causal, kv_len=kv_len)
    vis = np.isfinite(lse_ref)
    empty = int((~vis).sum())
    log(f"  rows without a visible key: {empty}")
    assert np.all(o[~vis] == 0.0), "rows without a visible key must give o = 0"
    assert np.all(np.isneginf(lse[~vis])), "rows without a visible key must give lse = -inf"
    if vis.any():
        bounds = None
        if w.dtype == "f32":
            bo, bl = f32_bounds(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype), w.scale, causal,
                                kv_len=kv_len)
            bounds = (bo[vis], bl[vis])
        compare(o[vis], lse[vis], o_ref[vis], lse_ref[vis], w.dtype, f"masked {causal} {kv_len}", bounds)
    return empty


W = si.Workload
CASES = [
    # (workload, causal, kv_len, splits)
    (W("m", 1, 3, 100, 700, 128, "bf16", True, "normal"), "bottom_right", None, 0),
    (W("m", 1, 3, 300, 200, 64, "bf16", True, "normal"), "bottom_right", None, 0),
    (W("m", 4, 2, 200, 500, 128, "bf16", True, "normal"), "top_left", [0, 1, 333, 500], 0),
    (W("m", 4, 2, 257, 500, 64, "bf16", False, "normal"), False, [17, 500, 64, 129], 0),
    (W("m", 2, 2, 130, 450, 128, "bf16", True, "normal"), "bottom_right", [450, 200], 0),
    (W("m", 2, 2, 130, 450, 128, "bf16", True, "normal"), "bottom_right", [450, 200], 5),
    (W("m", 2, 2, 64, 300, 64, "f32", True, "uniform01"), "bottom_right", [100, 300], 0),
    (W("m", 2, 2, 100, 300, 128, "f32", True, "uniform01"), "top_left", [300, 77], 3),
    (W("m", 4, 4, 1, 5000, 128, "bf16", True, "normal"), "bottom_right", [4000, 123, 5000, 0], 0),
    (W("m", 2, 4, 4, 3000, 64, "bf16", True, "normal"), "bottom_right", [3000, 1], 0),
    (W("m", 2, 2, 3, 900, 128, "f32", False, "normal"), False, [899, 2], 0),
    # key halves (few 128-row workgroups, long key ranges): a key length that
    # leaves the second set of waves one tile fewer, a single key, none
    (W("m", 2, 2, 300, 1000, 64, "bf16", True, "normal"), "bottom_right", [1000, 413], 0),
    (W("m", 3, 2, 200, 1100, 128, "bf16", True, "normal"), "top_left", [0, 1, 1100], 0),
    # 256-row widths (>= 256 workgroups of 256 rows): eight waves at d = 64,
    # 64 rows per wave at d = 128
    (W("m", 2, 128, 512, 700, 64, "bf16", True, "normal"), "bottom_right", [700, 301], 0),
    (W("m", 2, 128, 300, 260, 128, "bf16", True, "normal"), "top_left", [260, 1], 0),
    (W("m", 2, 128, 300, 700, 128, "bf16", True, "normal"), "bottom_right", [700, 333], 0),
    (W("m", 2, 128, 520, 300, 128, "bf16", True, "normal"), "bottom_right", [300, 0], 0),
    (W("m", 2, 128, 257, 1000, 128, "bf16", False, "normal"), False, [31, 1000], 0),
]


@pytest.mark.parametrize("w,causal,kv_len,splits", CASES,
                         ids=[f"{c[0].B}x{c[0].H}x{c[0].N}x{c[0].M}d{c[0].d}{c[0].dtype}-{c[1]}-{c[2]}-s{c[3]}"
                              for c in CASES])
def test_masks_match_oracle(w, causal, kv_len, splits):
    run_masked(w, causal, kv_len, splits)


def test_bottom_right_equals_top_left_when_square():
    import torch

    import online_softmax_10_amd as osa

    w = W("m", 2, 4, 333, 333, 128, "bf16", True, "normal")
    q, k, v = (to_device(a, "bf16") for a in si.make_qkv(w, 1))
    log("[gpu] bottom-right = top-left for N = M")
    o1, l1 = osa.fwd(q, k, v, causal=True)
    o2, l2 = osa.fwd(q, k, v, causal="bottom_right")
    o3, l3 = osa.fwd(q, k, v, causal=True, kv_len=torch.tensor([333, 333], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_bad_mask_arguments():
    import torch

    import online_softmax_10_amd as osa

    log("[gpu] masked binding argument checks")
    q = torch.zeros((2, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        osa.fwd(q, q, q, causal="diagonal")
    with pytest.raises(ValueError):
        osa.fwd(q, q, q, kv_len=torch.tensor([8, 8], dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        osa.fwd(q, q, q, kv_len=torch.tensor([8], dtype=torch.int32, device="cuda"))
