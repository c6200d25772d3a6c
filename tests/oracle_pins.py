"""Pins of the float64 oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` takes a loaded oracle library (``oracle.load()`` or a build of a
deliberately broken copy of ``oracle.c``) and raises AssertionError when the
oracle disagrees with:

* the values the pages print for their four worked examples (fixtures under
  ``tests/golden/``, each citing its page and example);
* identities the pages state (rows sum to 1, shift invariance of softmax,
  log p = z - LSE, the one-pass normaliser ending at the two-pass denominator,
  the stepwise / two-loop / blocked formulations ending at the same output);
* closed forms and special cases (one key, zero query, constant V, causal row
  0, identical keys, two-logit softmax = logistic function);
* library routines on tiny inputs (torch float64 softmax / logsumexp,
  scipy's logistic function).

No expected value here comes from the HIP path.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import recurrences as rec

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NEG_INF = float("-inf")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def close(a, b, tol: float, what: str) -> None:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    if a.size == 0:
        return
    err = float(np.max(np.abs(a - b)))
    assert np.all(np.isfinite(a)), f"{what}: non-finite values {a}"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}\n got {a}\n want {b}"


def _head(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x.reshape((1, 1) + x.shape)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- worked examples

def pin_w1_softmax(lib):
    g = golden("w1_softmax.json")
    x = np.array([g["logits"]])
    p = oracle.softmax(x, lib)[0]
    close(p, g["softmax"], g["tol_printed"], "W1 softmax vs printed")
    close(p.sum(), g["softmax_sum"], 1e-14, "W1 probabilities sum to 1")
    lse = oracle.logsumexp(x, lib)[0]
    close(math.exp(lse - g["max"]), g["sum_exp"], g["tol_printed"], "W1 sum of shifted exps")
    m, s = oracle.online_normalizer(x, lib)
    close(m[0], g["max"], 0.0, "W1 running max")
    close(s[0], g["sum_exp"], g["tol_printed"], "W1 one-pass denominator")


def pin_w2_cross_entropy(lib):
    g = golden("w2_cross_entropy.json")
    x = np.array([g["logits"]])
    c = g["label"]
    p = oracle.softmax(x, lib)[0]
    close(p[c], g["p_label"], g["tol_printed"], "W2 p_label")
    close(-math.log(p[c]), g["loss"], g["tol_printed"], "W2 loss from p")
    # log-softmax form: -log p_c = LSE(z) - z_c
    close(oracle.logsumexp(x, lib)[0] - x[0, c], g["loss"], g["tol_printed"], "W2 loss from LSE")


def pin_w3_attention(lib):
    g = golden("w3_attention.json")
    Q, K, V = (np.array(g[n]) for n in ("Q", "K", "V"))
    scale = 1.0 / math.sqrt(2.0)
    o, lse = oracle.attention(_head(Q), _head(K), _head(V), scale, False, lib)
    tol = g["tol_printed"]
    close(o[0, 0], g["O"], tol, "W3 output vs printed")
    S = np.array(g["QKt"]) * scale
    close(S, g["S"], 1e-4, "W3 scaled scores (fixture consistency)")
    P = oracle.softmax(S, lib)
    close(P, g["P"], tol, "W3 probabilities vs printed")
    close(np.exp(lse[0, 0] - S.max(axis=1)), g["row_sum_exp"], tol, "W3 row sums of shifted exps")
    # O = P V with the oracle's own probabilities (no other arithmetic involved)
    close(o[0, 0], P @ V, 1e-14, "W3 output equals P V")


def pin_w4_online_merge(lib):
    g = golden("w4_online_merge.json")
    x = np.array(g["scores"])
    V = np.array(g["V"])
    tol = g["tol_printed"]
    # scores given directly: q = e_0, k_j = x_j e_0, scale 1
    q = np.array([[1.0, 0.0]])
    k = np.stack([x, np.zeros_like(x)], axis=1)
    o, lse = oracle.attention(_head(q), _head(k), _head(V), 1.0, False, lib)
    st = g["standard"]
    close(o[0, 0, 0], st["output"], tol, "W4 standard output")
    close(oracle.softmax(x[None], lib)[0], st["probs"], tol, "W4 probabilities")
    close(math.exp(lse[0, 0, 0] - st["max"]), st["sum_exp"], tol, "W4 sum of exps")
    # every V row sums to 1, so the two output components sum to exactly 1
    close(o[0, 0, 0].sum(), 1.0, 1e-15, "W4 outputs sum to 1")
    # per-block states and the merge
    b1 = rec.block_state(x[:2], V[:2])
    b2 = rec.block_state(x[2:], V[2:])
    for (m, l, ov), want, name in ((b1, g["block1"], "block 1"), (b2, g["block2"], "block 2")):
        close(m, want["m"], 0.0, f"W4 {name} max")
        close(l, want["l"], tol, f"W4 {name} l")
        close(ov, want["o"], tol, f"W4 {name} o")
    mg = g["merged"]
    close(math.exp(b1[0] - mg["m"]), mg["scale_old"], tol, "W4 scale_old")
    m, l, ov = rec.merge_states(rec.merge_states((NEG_INF, 0.0, np.zeros(2)), b1), b2)
    close(m, mg["m"], 0.0, "W4 merged max")
    close(l, mg["l"], tol, "W4 merged l")
    close(ov, mg["output"], tol, "W4 merged output vs printed")
    close(ov, o[0, 0, 0], 1e-15, "W4 merged output equals the oracle")


# ---------------------------------------------------------------- softmax identities

def pin_softmax_identities(lib):
    import scipy.special
    import torch

    x = _rand((6, 37), 11, scale=4.0)
    p = oracle.softmax(x, lib)
    close(p.sum(axis=1), np.ones(6), 1e-14, "rows sum to 1")
    assert np.all(p > 0), "probabilities positive"
    # shift invariance (safe softmax equals softmax), also where e^x overflows
    close(oracle.softmax(x + 750.0, lib), p, 1e-13, "softmax(x + 750) = softmax(x)")
    close(oracle.logsumexp(x + 750.0, lib), oracle.logsumexp(x, lib) + 750.0, 1e-10,
          "LSE(x + c) = LSE(x) + c")
    # log p = z - LSE
    close(np.log(p), x - oracle.logsumexp(x, lib)[:, None], 1e-12, "log p = z - LSE")
    # library routines
    xt = torch.from_numpy(x)
    close(p, torch.softmax(xt, dim=-1).numpy(), 1e-15, "vs torch float64 softmax")
    close(oracle.logsumexp(x, lib), torch.logsumexp(xt, dim=-1).numpy(), 1e-13, "vs torch logsumexp")
    # two logits: p_0 is the logistic function of z_0 - z_1
    z = _rand((9, 2), 12, scale=5.0)
    close(oracle.softmax(z, lib)[:, 0], scipy.special.expit(z[:, 0] - z[:, 1]), 1e-15, "two-logit softmax")
    # equal logits -> uniform
    close(oracle.softmax(np.full((2, 7), 3.25), lib), np.full((2, 7), 1.0 / 7.0), 1e-16, "uniform")
    # one dominant logit
    close(oracle.softmax(np.array([[0.0, -800.0, -900.0]]), lib), [[1.0, 0.0, 0.0]], 0.0, "one-hot limit")


def pin_online_normalizer(lib):
    import torch

    x = _rand((5, 200), 13, scale=3.0)
    inc = np.cumsum(np.abs(_rand((1, 50), 14)), axis=1)       # max changes at every step
    dec = -np.cumsum(np.abs(_rand((1, 50), 15)), axis=1)      # max never changes
    one = np.array([[0.7]])
    for name, data in (("random", x), ("increasing", inc), ("decreasing", dec), ("single", one)):
        m, s = oracle.online_normalizer(data, lib)
        close(m, data.max(axis=1), 0.0, f"{name}: m_N is the max")
        # s_N equals the two-pass denominator sum_j e^{x_j - m_N}
        close(np.log(s) + m, oracle.logsumexp(data, lib), 1e-12, f"{name}: s_N = two-pass denominator")
        close(np.log(s) + m, torch.logsumexp(torch.from_numpy(data), -1).numpy(), 1e-12,
              f"{name}: s_N vs torch logsumexp")
    close(oracle.online_normalizer(one, lib)[1], [1.0], 0.0, "s_1 = 1")


# ---------------------------------------------------------------- attention

def _torch_attention(q, k, v, scale, causal):
    import torch

    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    if causal:
        N, M = s.shape[-2:]
        mask = torch.arange(M)[None, :] > torch.arange(N)[:, None]
        s = s.masked_fill(mask, float("-inf"))
    return (torch.matmul(torch.softmax(s, -1), vt).numpy(), torch.logsumexp(s, -1).numpy())


def pin_attention_brute_force(lib):
    cases = [(2, 3, 5, 7, 4, False), (2, 3, 5, 7, 4, True), (1, 2, 9, 4, 3, True),
             (1, 1, 4, 9, 2, True), (2, 2, 1, 6, 5, False)]
    for seed, (B, H, N, M, d, causal) in enumerate(cases):
        q = _rand((B, H, N, d), 100 + seed)
        k = _rand((B, H, M, d), 200 + seed)
        v = _rand((B, H, M, d), 300 + seed)
        scale = 0.37
        o, lse = oracle.attention(q, k, v, scale, causal, lib)
        to, tl = _torch_attention(q, k, v, scale, causal)
        close(o, to, 1e-13, f"attention vs torch {B,H,N,M,d,causal}")
        close(lse, tl, 1e-13, f"LSE vs torch {B,H,N,M,d,causal}")
        rows = np.array([B * H * N - 1, 0, (B * H * N) // 2], dtype=np.int64)
        ro, rl = oracle.attention_rows(q, k, v, scale, causal, rows, lib)
        close(ro, o.reshape(-1, d)[rows], 0.0, "row-sampled output equals full output")
        close(rl, lse.reshape(-1)[rows], 0.0, "row-sampled LSE equals full LSE")


def pin_attention_special_cases(lib):
    B, H, N, M, d = 2, 2, 6, 5, 3
    q = _rand((B, H, N, d), 21)
    k = _rand((B, H, M, d), 22)
    v = _rand((B, H, M, d), 23)
    sc = 0.61
    # one key: O = v_0, LSE = its score
    o, lse = oracle.attention(q, k[:, :, :1], v[:, :, :1], sc, False, lib)
    close(o, np.broadcast_to(v[:, :, :1], o.shape), 1e-15, "M=1: O = v_0")
    close(lse, sc * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]), 1e-14, "M=1: LSE = score")
    for causal in (False, True):
        vis = np.array([min(M, i + 1) if causal else M for i in range(N)])
        # zero query: uniform weights over the visible keys
        o, lse = oracle.attention(np.zeros_like(q), k, v, sc, causal, lib)
        want = np.stack([v[:, :, :n].mean(axis=2) for n in vis], axis=2)
        close(o, want, 1e-15, f"q=0: O = mean of visible V (causal={causal})")
        close(lse, np.broadcast_to(np.log(vis), lse.shape), 1e-15, f"q=0: LSE = log #visible (causal={causal})")
        # identical keys: uniform again, LSE = score + log #visible
        kk = np.broadcast_to(k[:, :, :1], k.shape).copy()
        o2, lse2 = oracle.attention(q, kk, v, sc, causal, lib)
        close(o2, want, 1e-14, f"identical keys: O = mean of visible V (causal={causal})")
        # constant V rows: O is that constant
        o3, _ = oracle.attention(q, k, np.ones_like(v) * 2.5, sc, causal, lib)
        close(o3, np.full_like(o3, 2.5), 1e-14, f"V = 2.5: O = 2.5 (causal={causal})")
        # affine in V (weights sum to 1)
        o4, _ = oracle.attention(q, k, 3.0 * v - 1.25, sc, causal, lib)
        o5, l5 = oracle.attention(q, k, v, sc, causal, lib)
        close(o4, 3.0 * o5 - 1.25, 1e-13, f"O(aV+b) = aO(V)+b (causal={causal})")
        # adding one vector w to every key shifts each row's scores by sc*<q_i,w>
        w = _rand((B, H, 1, d), 24)
        o6, l6 = oracle.attention(q, k + w, v, sc, causal, lib)
        close(o6, o5, 1e-13, f"key shift leaves O (causal={causal})")
        close(l6, l5 + sc * np.einsum("bhnd,bhd->bhn", q, w[:, :, 0]), 1e-13, f"key shift moves LSE (causal={causal})")
    # causal row 0 sees only key 0
    o, lse = oracle.attention(q, k, v, sc, True, lib)
    close(o[:, :, 0], v[:, :, 0], 1e-15, "causal row 0: O = v_0")
    close(lse[:, :, 0], sc * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-14, "causal row 0: LSE")
    # causal row i equals non-causal attention over keys 0..i
    for i in range(N):
        n = min(M, i + 1)
        oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], sc, False, lib)
        close(o[:, :, i:i + 1], oi, 1e-15, f"causal row {i} = prefix attention")
        close(lse[:, :, i:i + 1], li, 1e-15, f"causal row {i} LSE = prefix LSE")
    # permuting keys and values together changes nothing (non-causal)
    perm = np.random.default_rng(25).permutation(M)
    o7, l7 = oracle.attention(q, k[:, :, perm], v[:, :, perm], sc, False, lib)
    o8, l8 = oracle.attention(q, k, v, sc, False, lib)
    close(o7, o8, 1e-14, "key permutation")
    close(l7, l8, 1e-14, "key permutation LSE")
    # heads are independent
    o9, l9 = oracle.attention(q[1:, 1:], k[1:, 1:], v[1:, 1:], sc, False, lib)
    close(o9, o8[1:, 1:], 0.0, "heads independent")
    # large logits: the max shift prevents overflow
    o10, l10 = oracle.attention(q * 40.0, k * 40.0, v, 1.0, True, lib)
    assert np.all(np.isfinite(o10)) and np.all(np.isfinite(l10)), "large logits stay finite"
    to, tl = _torch_attention(q * 40.0, k * 40.0, v, 1.0, True)
    close(o10, to, 1e-12, "large logits vs torch")
    close(l10, tl, 1e-10, "large logits LSE vs torch")


def pin_formulations_agree(lib):
    B, H, N, M, d = 1, 2, 7, 9, 3
    q = _rand((B, H, N, d), 31)
    k = _rand((B, H, M, d), 32)
    v = _rand((B, H, M, d), 33)
    sc = 0.8
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, sc, causal, lib)
        for Br in (1, 2, 3, 5, N):
            for Bc in (1, 2, 3, 5, 17):
                ob, lb = rec.blocked_attention(q, k, v, sc, causal, Br, Bc)
                close(ob, o, 1e-12, f"blocked Br={Br} Bc={Bc} causal={causal}")
                close(lb, lse, 1e-12, f"blocked LSE Br={Br} Bc={Bc} causal={causal}")
        for splits in (1, 2, 4, 9):
            os_, ls_ = rec.split_merge_attention(q, k, v, sc, causal, splits)
            close(os_, o, 1e-12, f"split-merge S={splits} causal={causal}")
            close(ls_, lse, 1e-12, f"split-merge LSE S={splits} causal={causal}")
        for i in range(N):
            n = min(M, i + 1) if causal else M
            x = sc * (k[0, 0, :n] @ q[0, 0, i])
            a2, g2, s2 = rec.two_loop_row(x, v[0, 0, :n])
            a3, g3, s3 = rec.stepwise_normalised_row(x, v[0, 0, :n])
            close(a2, o[0, 0, i], 1e-13, f"two-loop row {i} causal={causal}")
            close(a3, o[0, 0, i], 1e-13, f"stepwise row {i} causal={causal}")
            close(g2 + math.log(s2), lse[0, 0, i], 1e-13, f"two-loop g_M + log s_M row {i}")
            close(g3 + math.log(s3), lse[0, 0, i], 1e-13, f"stepwise g_M + log s_M row {i}")


def pin_cross_entropy(lib):
    # The worked example: logits [2, 1, 0.1], class 0.
    g = golden("w2_cross_entropy.json")
    loss, lse, mean = oracle.cross_entropy(np.array([g["logits"]]), [g["label"]], lib)
    close(loss[0], g["loss"], g["tol_printed"], "W2 cross-entropy vs printed")
    close(mean, g["loss"], g["tol_printed"], "W2 batch mean of one row")
    # torch's float64 cross-entropy on small random batches (per row and mean).
    import torch
    import torch.nn.functional as F

    for seed, (rows, n, spread) in enumerate(((7, 5, 3.0), (4, 33, 10.0), (3, 1, 1.0))):
        x = _rand((rows, n), 100 + seed, spread)
        lab = np.random.default_rng(200 + seed).integers(0, n, size=rows)
        loss, lse, mean = oracle.cross_entropy(x, lab, lib)
        xt, lt = torch.from_numpy(x), torch.from_numpy(lab)
        close(loss, F.cross_entropy(xt, lt, reduction="none").numpy(), 1e-12, f"torch cross_entropy {rows}x{n}")
        close(mean, float(F.cross_entropy(xt, lt, reduction="mean")), 1e-12, f"torch mean {rows}x{n}")
        close(lse, torch.logsumexp(xt, dim=1).numpy(), 1e-12, f"torch logsumexp {rows}x{n}")
    # Closed forms: equal logits give log n for any label; two classes give the
    # softplus of the logit gap; a dominant label logit gives ~0 without overflow.
    for n in (1, 2, 3, 10, 1000):
        x = np.full((3, n), 7.25)
        loss, _, _ = oracle.cross_entropy(x, [0, n - 1, n // 2], lib)
        close(loss, [math.log(n)] * 3, 1e-12, f"uniform logits n={n}")
    for a, b in ((0.0, 0.0), (2.0, -1.0), (-3.5, 4.25), (30.0, -30.0)):
        loss, _, _ = oracle.cross_entropy(np.array([[a, b]]), [0], lib)
        close(loss[0], math.log1p(math.exp(b - a)), 1e-12, f"two-class softplus {a},{b}")
    loss, lse, _ = oracle.cross_entropy(np.array([[1000.0, 0.0, -5.0]]), [0], lib)
    close(loss[0], 0.0, 1e-300 + 1e-15, "dominant label, huge logit")
    close(lse[0], 1000.0, 1e-12, "LSE of a dominant huge logit")
    # Shift invariance of the loss; the LSE moves with the shift.
    x = _rand((5, 17), 7, 2.0)
    lab = np.arange(5) * 3
    l0, s0, _ = oracle.cross_entropy(x, lab, lib)
    l1, s1, _ = oracle.cross_entropy(x + 750.0, lab, lib)
    close(l1, l0, 1e-9, "loss shift invariance")
    close(s1 - 750.0, s0, 1e-9, "LSE shift")
    close(l0, s0 - x[np.arange(5), lab], 1e-12, "loss = LSE - z_label")
    # A label outside [0, n) has no log probability.
    loss, _, _ = oracle.cross_entropy(np.zeros((3, 4)), [-1, 4, 2], lib)
    assert math.isnan(loss[0]) and math.isnan(loss[1]) and abs(loss[2] - math.log(4)) < 1e-12, loss


def _torch_masked(q, k, v, scale, mode, kv_len):
    """softmax(masked scores) V and LSE with torch float64, rows with a visible key only."""
    import torch

    qt, kt, vt = (torch.from_numpy(a) for a in (q, k, v))
    B, H, N, d = q.shape
    M = k.shape[2]
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    i = torch.arange(N).view(N, 1)
    j = torch.arange(M).view(1, M)
    allow = torch.ones(B, 1, N, M, dtype=torch.bool)
    if mode == "top_left":
        allow &= (j <= i)
    elif mode == "bottom_right":
        allow &= (j <= i + (M - N))
    if kv_len is not None:
        allow &= (j.view(1, 1, 1, M) < torch.tensor(kv_len).view(B, 1, 1, 1))
    s = s.masked_fill(~allow, float("-inf"))
    any_visible = allow.expand(B, H, N, M).any(dim=-1)
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(torch.nan_to_num(p, nan=0.0), vt)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy(), any_visible.numpy()


def pin_attention_masks(lib):
    # torch float64 with explicit boolean masks on small random problems.
    cases = [(2, 2, 5, 9, 4, "bottom_right", None), (2, 2, 9, 5, 4, "bottom_right", None),
             (2, 1, 7, 7, 3, "top_left", [3, 7]), (3, 2, 6, 11, 4, False, [0, 5, 11]),
             (2, 2, 8, 6, 4, "bottom_right", [2, 6]), (1, 3, 4, 13, 5, "top_left", [9])]
    for n, (B, H, N, M, d, mode, kl) in enumerate(cases):
        q, k, v = _rand((B, H, N, d), 50 + n), _rand((B, H, M, d), 60 + n), _rand((B, H, M, d), 70 + n)
        scale = 0.7
        o, lse = oracle.attention(q, k, v, scale, mode, lib, kv_len=kl)
        ro, rl, vis = _torch_masked(q, k, v, scale, mode, kl)
        close(o[vis], ro[vis], 1e-12, f"masked attention O vs torch, case {n}")
        close(lse[vis], rl[vis], 1e-12, f"masked attention LSE vs torch, case {n}")
        assert np.all(o[~vis] == 0.0) and np.all(np.isneginf(lse[~vis])), f"empty rows, case {n}"
    # Special cases that reduce to the plain definitions.
    q, k, v = _rand((2, 2, 6, 4), 80), _rand((2, 2, 6, 4), 81), _rand((2, 2, 6, 4), 82)
    o1, l1 = oracle.attention(q, k, v, 0.5, True, lib)
    o2, l2 = oracle.attention(q, k, v, 0.5, "bottom_right", lib)
    close(o2, o1, 0.0, "bottom-right = top-left when N = M")
    close(l2, l1, 0.0, "bottom-right LSE = top-left LSE when N = M")
    o3, l3 = oracle.attention(q, k, v, 0.5, False, lib, kv_len=[6, 6])
    o4, l4 = oracle.attention(q, k, v, 0.5, False, lib)
    close(o3, o4, 0.0, "key lengths of M = no key mask")
    close(l3, l4, 0.0, "key lengths of M = no key mask (LSE)")
    o5, l5 = oracle.attention(q, k, v, 0.5, False, lib, kv_len=[4, 2])
    for b, L in enumerate((4, 2)):
        ob, lb = oracle.attention(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.5, False, lib)
        close(o5[b:b + 1], ob, 1e-14, f"key length {L} = keys sliced")
        close(l5[b:b + 1], lb, 1e-14, f"key length {L} = keys sliced (LSE)")
    # Bottom-right, N > M: the first N - M rows see no key.
    q, k, v = _rand((1, 1, 7, 3), 90), _rand((1, 1, 4, 3), 91), _rand((1, 1, 4, 3), 92)
    o, l = oracle.attention(q, k, v, 1.0, "bottom_right", lib)
    assert np.all(o[0, 0, :3] == 0.0) and np.all(np.isneginf(l[0, 0, :3]))
    for i in range(3, 7):
        oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, :i - 2], v[:, :, :i - 2], 1.0, False, lib)
        close(o[0, 0, i], oi[0, 0, 0], 1e-14, f"bottom-right row {i} = keys 0..{i - 3}")
        close(l[0, 0, i], li[0, 0, 0], 1e-14, f"bottom-right row {i} LSE")


def pin_attention_bias(lib):
    # Additive score bias: softmax(scale * Q K^T + bias) V.
    import torch

    rng = np.random.default_rng(95)
    B, H, N, M, d = 2, 3, 5, 7, 4
    q, k, v = _rand((B, H, N, d), 96), _rand((B, H, M, d), 97), _rand((B, H, M, d), 98)
    bias = rng.standard_normal((B, H, N, M)) * 2.0
    # Q = 0: the scores are the bias alone, so O is the e^bias-weighted mean of
    # the values and LSE = log sum_j e^bias.
    o, lse = oracle.attention(np.zeros_like(q), k, v, 0.7, False, lib, bias=bias)
    w = np.exp(bias)
    close(o, np.einsum("bhij,bhjd->bhid", w, v) / w.sum(-1, keepdims=True), 1e-14, "bias-only weights")
    close(lse, np.log(w.sum(-1)), 1e-14, "bias-only LSE")
    # A constant per row changes nothing but the LSE, by that constant.
    o0, l0 = oracle.attention(q, k, v, 0.7, False, lib)
    row_c = rng.standard_normal((B, H, N, 1)) * 5.0
    o1, l1 = oracle.attention(q, k, v, 0.7, False, lib, bias=np.broadcast_to(row_c, (B, H, N, M)))
    close(o1, o0, 1e-13, "row-constant bias leaves O")
    close(l1, l0 + row_c[..., 0], 1e-13, "row-constant bias shifts LSE")
    # -inf on keys >= L_b is the key-length mask.
    L = [3, 7]
    neg = np.zeros((B, H, N, M))
    for b, Lb in enumerate(L):
        neg[b, :, :, Lb:] = -np.inf
    o2, l2 = oracle.attention(q, k, v, 0.7, "bottom_right", lib, bias=neg)
    o3, l3 = oracle.attention(q, k, v, 0.7, "bottom_right", lib, kv_len=L)
    close(o2, o3, 0.0, "-inf bias = key lengths")
    close(l2, l3, 0.0, "-inf bias = key lengths (LSE)")
    # A bias broadcast over batch and heads = the same bias written out.
    b2 = rng.standard_normal((N, M))
    o4, l4 = oracle.attention(q, k, v, 0.7, True, lib, bias=b2)
    o5, l5 = oracle.attention(q, k, v, 0.7, True, lib, bias=np.ascontiguousarray(np.broadcast_to(b2, (B, H, N, M))))
    close(o4, o5, 0.0, "broadcast bias = expanded bias")
    close(l4, l5, 0.0, "broadcast bias = expanded bias (LSE)")
    # A row whose scores are all -inf: o = 0, LSE = -inf; the other rows as
    # with that row's bias absent.
    b3 = bias.copy()
    b3[1, 2, 3, :] = -np.inf
    o6, l6 = oracle.attention(q, k, v, 0.7, False, lib, bias=b3)
    o7, l7 = oracle.attention(q, k, v, 0.7, False, lib, bias=bias)
    assert np.all(o6[1, 2, 3] == 0.0) and np.isneginf(l6[1, 2, 3]), "all -inf row"
    keep = np.ones((B, H, N), dtype=bool)
    keep[1, 2, 3] = False
    close(o6[keep], o7[keep], 0.0, "other rows unchanged by one -inf row")
    # torch float64 brute force, with the causal masks.
    for mode in (True, "bottom_right"):
        o8, l8 = oracle.attention(q, k, v, 0.7, mode, lib, bias=bias)
        s = 0.7 * torch.matmul(torch.from_numpy(q), torch.from_numpy(k).transpose(-1, -2).contiguous())
        s = s + torch.from_numpy(bias)
        i = torch.arange(N)[:, None]
        j = torch.arange(M)[None, :]
        off = 0 if mode is True else M - N
        s = s.masked_fill(j > i + off, float("-inf"))
        ro = torch.matmul(torch.softmax(s, -1), torch.from_numpy(v))
        close(o8, ro.numpy(), 1e-13, f"biased attention vs torch ({mode})")
        close(l8, torch.logsumexp(s, -1).numpy(), 1e-13, f"biased LSE vs torch ({mode})")


ALL_PINS = [
    pin_w1_softmax,
    pin_w2_cross_entropy,
    pin_cross_entropy,
    pin_w3_attention,
    pin_w4_online_merge,
    pin_softmax_identities,
    pin_online_normalizer,
    pin_attention_brute_force,
    pin_attention_special_cases,
    pin_attention_masks,
    pin_attention_bias,
    pin_formulations_agree,
]
