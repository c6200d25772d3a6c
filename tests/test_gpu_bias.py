"""GPU parity of the additive score bias (attn_fwd_masked through the C ABI)
against the float64 oracle: full, broadcast and padded (M % 4 != 0) bias
layouts, both head sizes and dtypes, decode shapes, forced splits, key
lengths and causal masks combined with the bias, -inf entries and a row whose
scores are all -inf (o = 0, lse = -inf), and a large distance penalty."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import compare, f32_bounds, log, to_device

pytestmark = pytest.mark.gpu

W = si.Workload


def run_bias(w, causal, bshape, kind="normal", kv_len=None, splits=0, neg_inf_frac=0.0, dead=None, seed=0):
    import torch

    import online_softmax_10_amd as osa

    q, k, v = si.make_qkv(w, seed)
    bias = si.make_bias(bshape, seed + 100, kind, neg_inf_frac)
    if dead is not None:
        bias[dead] = -np.inf
    log(f"[gpu] bias B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} causal={causal} bias{bshape} {kind} "
        f"kv_len={kv_len} splits={splits} -inf frac={neg_inf_frac} dead={dead}")
    qd, kd, vd = (to_device(a, w.dtype) for a in (q, k, v))
    bd = torch.from_numpy(bias).cuda()
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    o, lse = osa.fwd_splits(qd, kd, vd, scale=w.scale, causal=causal, num_splits=splits, kv_len=kl, bias=bd)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype),
                                      w.scale, causal, kv_len=kv_len, bias=bias.astype(np.float64))
    vis = np.isfinite(lse_ref)
    log(f"  rows with no finite score: {int((~vis).sum())}")
    assert np.all(o[~vis] == 0.0), "rows with no finite score must give o = 0"
    assert np.all(np.isneginf(lse[~vis])), "rows with no finite score must give lse = -inf"
    bounds = None
    if w.dtype == "f32":
        bo, bl = f32_bounds(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype), w.scale, causal,
                            kv_len=kv_len, bias=bias.astype(np.float64))
        bounds = (bo[vis], bl[vis])
    compare(o[vis], lse[vis], o_ref[vis], lse_ref[vis], w.dtype, f"bias {bshape} {causal}", bounds)
    return int((~vis).sum())


CASES = [
    # (workload, causal, bias shape, kind, kv_len, splits, -inf fraction)
    (W("b", 2, 3, 300, 520, 128, "bf16", True, "normal"), "bottom_right", (2, 3, 300, 520), "normal", None, 0, 0.0),
    (W("b", 2, 2, 257, 257, 64, "bf16", False, "normal"), False, (257, 257), "normal", None, 0, 0.0),
    (W("b", 2, 2, 200, 333, 128, "bf16", True, "normal"), "top_left", (2, 1, 200, 333), "normal", [333, 150], 0, 0.1),
    (W("b", 2, 4, 3, 2000, 128, "bf16", False, "normal"), False, (2, 1, 3, 2000), "normal", [2000, 5], 0, 0.0),
    (W("b", 1, 4, 1, 4096, 64, "bf16", False, "normal"), False, (1, 4, 1, 4096), "normal", None, 0, 0.0),
    (W("b", 1, 2, 130, 1000, 128, "bf16", True, "normal"), "bottom_right", (1, 2, 1, 1000), "normal", None, 3, 0.0),
    (W("b", 1, 2, 130, 1000, 64, "bf16", False, "normal"), False, (130, 1000), "normal", [700], 4, 0.3),
    (W("b", 1, 1, 256, 256, 64, "f32", False, "uniform01"), False, (1, 1, 256, 256), "normal", None, 0, 0.0),
    (W("b", 2, 2, 100, 301, 128, "f32", True, "normal"), "bottom_right", (2, 2, 100, 301), "normal", None, 2, 0.2),
    (W("b", 1, 8, 1024, 1024, 128, "bf16", True, "normal"), True, (1, 8, 1024, 1024), "distance", None, 0, 0.0),
    # key halves with a bias (d = 64, few 128-row tiles, long key ranges)
    (W("b", 2, 2, 300, 1000, 64, "bf16", True, "normal"), "bottom_right", (2, 2, 300, 1000), "normal", [1000, 555], 0,
     0.1),
    (W("b", 1, 4, 200, 900, 64, "bf16", False, "normal"), False, (1, 4, 200, 900), "distance", None, 0, 0.0),
    (W("b", 1, 2, 129, 1025, 64, "bf16", True, "normal"), True, (1, 2, 1, 1025), "normal", None, 0, 0.0),
]


@pytest.mark.parametrize("w,causal,bshape,kind,kv_len,splits,frac", CASES,
                         ids=[f"{c[0].B}x{c[0].H}x{c[0].N}x{c[0].M}d{c[0].d}{c[0].dtype}-{c[1]}-b{'x'.join(map(str, c[2]))}"
                              f"-{c[3]}-{c[4]}-s{c[5]}-f{c[6]}" for c in CASES])
def test_bias_matches_oracle(w, causal, bshape, kind, kv_len, splits, frac):
    run_bias(w, causal, bshape, kind, kv_len, splits, frac)


@pytest.mark.parametrize("dtype,d,M", [("bf16", 128, 150), ("bf16", 64, 150), ("f32", 64, 150), ("bf16", 64, 1000)])
def test_bias_dead_row(dtype, d, M):
    # One row's bias is -inf at every key: o = 0, lse = -inf for it alone
    # (M = 1000 at d = 64: the key-halves kernel, both sets without a key).
    w = W("b", 2, 2, 70, M, d, dtype, False, "normal")
    assert run_bias(w, False, (2, 2, 70, M), dead=(1, 0, 33)) == 1


def test_zero_bias_equals_no_bias():
    import torch

    import online_softmax_10_amd as osa

    w = W("b", 2, 4, 333, 333, 128, "bf16", True, "normal")
    q, k, v = (to_device(a, "bf16") for a in si.make_qkv(w, 3))
    log("[gpu] zero bias = no bias (four-wave kernel with and without the bias path)")
    o1, l1 = osa.fwd(q, k, v, causal=True, bias=torch.zeros((333, 333), dtype=torch.float32, device="cuda"))
    o2, l2 = osa.fwd_splits(q, k, v, causal=True, num_splits=1)
    torch.cuda.synchronize()
    # The bias path rounds c*s before the shift (the plain path fuses both in
    # one FMA).  That can move a lazily kept shift, and P is rounded to bf16
    # against its shift (2^-9 relative), so the two paths agree to the bf16
    # rounding of P, well inside the oracle tolerances (5e-3 LSE, 1e-2 O).
    dl = (l1 - l2).abs().max().item()
    do = (o1.float() - o2.float()).abs().max().item()
    log(f"  max |dlse| {dl:.2e}  max |do| {do:.2e}")
    assert dl <= 2e-3 and do <= 8e-3
