"""attn_fwd_masked_noalloc (through the C ABI) against attn_fwd_masked: the
same plans and kernels with the split partials in the library's static device
scratch instead of a stream-ordered allocation.  Two calls in a row, the
second smaller, on every plan that uses the scratch (decode splits, four-wave
bf16 splits, fp32 splits, masks and a bias) and on a single pass (which uses
none): outputs equal bit for bit, and the first case also within the rule
against the oracle."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import compare, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_10_amd as osa

    osa.lib()
    yield


def _both(w, seed, splits, causal=None, kv_len=None, bias=None):
    import torch

    import online_softmax_10_amd as osa

    q, k, v = si.make_qkv(w, seed)
    qd, kd, vd = (to_device(a, w.dtype) for a in (q, k, v))
    causal = w.causal if causal is None else causal
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    plan = osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype, splits)
    log(f"[gpu] noalloc B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} causal={causal} splits={splits} "
        f"kv_len={kv_len} bias={bias is not None} plan={plan}")
    # Outputs allocated up front: the no-allocation call itself allocates nothing.
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o1 = torch.full((w.B, w.H, w.N, w.d), 7.0, dtype=tdtype, device="cuda")
    l1 = torch.full((w.B, w.H, w.N), 7.0, dtype=torch.float32, device="cuda")
    osa.fwd_noalloc(qd, kd, vd, scale=w.scale, causal=causal, num_splits=splits, out=o1, lse=l1, kv_len=kl, bias=bd)
    o2, l2 = osa.fwd_splits(qd, kd, vd, scale=w.scale, causal=causal, num_splits=splits, kv_len=kl, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "o differs from attn_fwd_masked"
    assert torch.equal(l1, l2), "lse differs from attn_fwd_masked"
    return (q, k, v), o1, l1


CASES = [
    # (large, small): the second call is smaller than the first
    ((si.Workload("na", 8, 16, 1, 8192, 128, "bf16", False, "normal"), 0),
     (si.Workload("na", 2, 4, 3, 3000, 128, "bf16", True, "normal"), 0)),          # decode splits
    ((si.Workload("na", 2, 3, 200, 4000, 128, "bf16", True, "normal"), 7),
     (si.Workload("na", 1, 2, 130, 700, 64, "bf16", False, "normal"), 3)),          # four-wave splits
    ((si.Workload("na", 1, 2, 130, 700, 64, "f32", False, "uniform01"), 16),
     (si.Workload("na", 1, 1, 40, 200, 64, "f32", True, "normal"), 2)),             # fp32 splits
    ((si.Workload("na", 4, 8, 1024, 1024, 64, "bf16", False, "normal"), 1),
     (si.Workload("na", 1, 2, 100, 90, 128, "bf16", True, "normal"), 1)),           # single pass
]


@pytest.mark.parametrize("pair", CASES, ids=["decode", "bf16-splits", "f32-splits", "single"])
def test_noalloc_matches_attn_fwd_masked(pair):
    for i, (w, splits) in enumerate(pair):
        (q, k, v), o, lse = _both(w, 30 + i, splits)
        if i == 0 and w.N * w.B * w.H <= 8192:
            o_ref, l_ref = oracle.attention(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype),
                                            w.scale, w.causal)
            compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
                    w.dtype, "noalloc vs oracle")


def test_noalloc_masks_and_bias():
    w = si.Workload("na", 2, 2, 130, 450, 128, "bf16", True, "normal")
    _both(w, 40, 5, causal="bottom_right", kv_len=[450, 200])
    bias = si.make_bias((w.N, w.M), 8)
    _both(w.with_shape(N=100, M=300), 41, 4, causal=True, bias=bias[:100, :300].copy())


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    import torch

    import online_softmax_10_amd as osa

    q = torch.zeros((1, 1, 300, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 300000, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(osa.AttnError) as e:
        osa.fwd_noalloc(q, k, k, num_splits=256)
    assert e.value.code == -11
