"""The library runs on the caller's stream: calls on a side stream ordered by
that stream alone (no host synchronisation between producer, call and
consumer), calls on two streams at once, and HIP graph capture of the
single-pass attention and the row softmax (replayed with eager work and
synchronisations between replays, every replay checked).  Each result is
compared bit for bit with the same call on the default stream: the kernels
are deterministic."""

import numpy as np
import pytest

import seeded_inputs as si
from parity import log, to_device

pytestmark = pytest.mark.gpu


def _inputs(w, seed):
    return tuple(to_device(a, w.dtype) for a in si.make_qkv(w, seed))


def test_side_stream_orders_producer_call_consumer():
    import torch

    import online_softmax_10_amd as osa

    for w, splits in ((si.Workload("s", 2, 8, 700, 900, 128, "bf16", True, "normal"), 0),
                      (si.Workload("s", 1, 4, 200, 3000, 64, "bf16", False, "normal"), 5),
                      (si.Workload("s", 2, 16, 1, 4000, 128, "bf16", False, "normal"), 0)):
        log(f"[gpu] side stream B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} splits={splits} "
            f"plan={osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype, splits)}")
        q, k, v = _inputs(w, 3)
        o_ref, l_ref = osa.fwd_splits(q, k, v, causal=w.causal, num_splits=splits)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            # producer (a copy on the side stream), the call, a consumer, all
            # ordered by the side stream only
            q2 = q.clone()
            o, lse = osa.fwd_splits(q2, k, v, causal=w.causal, num_splits=splits)
            o_sum = o.float().sum()
        s.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        assert torch.isfinite(o_sum)

    x = torch.from_numpy(si.make_rows(4096, 1000, seed=5)).cuda()
    labels = torch.randint(0, 1000, (4096,), device="cuda", generator=torch.Generator("cuda").manual_seed(1))
    y_ref, lse_ref = osa.online_softmax(x, return_lse=True)
    loss_ref, _, mean_ref = osa.softmax_xent(x, labels)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        x2 = x.clone()
        y, lse = osa.online_softmax(x2, return_lse=True)
        loss, _, mean = osa.softmax_xent(x2, labels)
    s.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(lse, lse_ref)
    assert torch.equal(loss, loss_ref) and torch.equal(mean, mean_ref)


def test_two_streams_at_once():
    import torch

    import online_softmax_10_amd as osa

    w = si.Workload("s", 2, 16, 1024, 1024, 128, "bf16", True, "normal")
    inputs = [_inputs(w, 10 + i) for i in range(2)]
    refs = [osa.fwd(*qkv, causal=True) for qkv in inputs]
    torch.cuda.synchronize()
    log("[gpu] two streams at once")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs[i] = osa.fwd(*inputs[i], causal=True)
        for s in streams:
            s.synchronize()
        for i in range(2):
            assert torch.equal(outs[i][0], refs[i][0]) and torch.equal(outs[i][1], refs[i][1]), (rep, i)


@pytest.mark.parametrize("shape", [(2, 8, 512, 768, 128), (1, 4, 512, 1024, 64)], ids=["four_wave", "key_halves"])
def test_graph_capture_and_replay(shape):
    import torch

    import online_softmax_10_amd as osa

    B, H, N, M, d = shape
    w = si.Workload("g", B, H, N, M, d, "bf16", True, "normal")
    q, k, v = _inputs(w, 20)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    x = torch.from_numpy(si.make_rows(512, 2048, seed=21)).cuda()
    y = torch.empty_like(x)
    log(f"[gpu] graph capture: attention plan {osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype, 1)} + online_softmax")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            osa.fwd_splits(q, k, v, causal=True, num_splits=1, out=o, lse=lse)
            osa.online_softmax(x, out=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        osa.fwd_splits(q, k, v, causal=True, num_splits=1, out=o, lse=lse)
        osa.online_softmax(x, out=y)
    for rep in range(4):
        # eager work between replays: new inputs written in place
        qn, kn, vn = _inputs(w, 30 + rep)
        q.copy_(qn)
        k.copy_(kn)
        v.copy_(vn)
        x.copy_(torch.from_numpy(si.make_rows(512, 2048, seed=40 + rep)).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = osa.fwd_splits(q, k, v, causal=True, num_splits=1)
        y_ref = osa.online_softmax(x)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep}: attention"
        assert torch.equal(y, y_ref), f"replay {rep}: online_softmax"
    del g
