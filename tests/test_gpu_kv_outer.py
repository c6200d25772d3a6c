"""GPU parity of attn_fwd_kv_outer (the key/value-outer loop order, row state
through HBM after every key block) against the float64 oracle."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import compare, log, to_device

pytestmark = pytest.mark.gpu

W = si.Workload
CASES = [
    W("kvo", 1, 2, 300, 300, 128, "bf16", True, "normal"),
    W("kvo", 2, 2, 257, 513, 64, "bf16", False, "normal"),
    W("kvo", 1, 1, 130, 1000, 128, "bf16", True, "normal"),
    W("kvo", 1, 2, 500, 100, 64, "bf16", True, "normal"),
    W("kvo", 1, 2, 200, 700, 128, "bf16", True, "normal_qk3"),
    W("kvo", 2, 1, 64, 64, 128, "bf16", False, "normal"),
]


@pytest.mark.parametrize("w", CASES, ids=[f"{w.B}x{w.H}x{w.N}x{w.M}d{w.d}{'c' if w.causal else ''}{w.dist}"
                                          for w in CASES])
def test_kv_outer_matches_oracle(w):
    import torch

    import online_softmax_10_amd as osa

    q, k, v = si.make_qkv(w, 3)
    log(f"[gpu] kv-outer B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} causal={w.causal} {w.dist}")
    qd, kd, vd = (to_device(a, "bf16") for a in (q, k, v))
    o, lse = osa.fwd_kv_outer(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(si.to_f64(q, "bf16"), si.to_f64(k, "bf16"), si.to_f64(v, "bf16"),
                                      w.scale, w.causal)
    compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
            "bf16", f"kv-outer {w.B}x{w.H}x{w.N}x{w.M}")


def test_kv_outer_rejects_fp32():
    import torch

    import online_softmax_10_amd as osa

    q = torch.zeros((1, 1, 8, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        osa.fwd_kv_outer(q, q, q)
