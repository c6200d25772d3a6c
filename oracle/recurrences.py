"""The pages' other formulations of attention, in plain float64 Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Small inputs only:
these are element-by-element loops written for reading, not for speed.  They
exist to cross-check the plain definition in ``oracle.c`` (which is what the
HIP path is compared against) and to pin the pages' worked examples.

Notation follows the pages: scores x (or s), running max g (or m), running
exponential sum s (or l), accumulated output A' (normalised) or o~
(unnormalised).
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def _exp(t: float) -> float:
    return 0.0 if t == NEG_INF else math.exp(t)


def two_loop_row(x, V):
    """Attention for one query row from its scores x[0..M-1] and V [M, d].

    Loop 1 carries the normaliser (g, s) of the scores seen so far -- their
    maximum and their sum of e^{x - g} -- from the empty prefix (-inf, 0),
    one score at a time: g' = max(g, x_m), s' = s e^{g - g'} + e^{x_m - g'}.
    Loop 2 sums the normalised weights e^{x_m - g_M} / s_M times V[m,:].
    Source: "Online Softmax and Flash Attention" page, eq. (10)-(13) (loop 1)
    and eq. (14)-(15) (loop 2).
    Returns (A_M, g_M, s_M).
    """
    x = [float(t) for t in x]
    V = np.asarray(V, dtype=np.float64)
    g, s = NEG_INF, 0.0
    for xm in x:
        g_next = max(g, xm)
        if g_next == NEG_INF:
            continue  # only -inf so far: the prefix stays empty
        s = s * _exp(g - g_next) + _exp(xm - g_next)
        g = g_next
    A = np.zeros(V.shape[1])
    for m in range(len(x)):
        A = A + (_exp(x[m] - g) / s) * V[m]
    return A, g, s


def stepwise_normalised_row(x, V):
    """The single fused loop with a normalised accumulator A'.

    The state (g, s, A') of the scores seen so far -- maximum, sum of
    e^{x - g}, and the attention row over just those keys -- starts empty
    ((-inf, 0, 0)) and takes one key at a time: with g' = max(g, x_m) and
    s' = s e^{g - g'} + e^{x_m - g'}, the old row keeps the weight
    s e^{g - g'} / s' and V[m] gets e^{x_m - g'} / s'.  A'_M is the row.
    Source: "Online Softmax and Flash Attention" page, eq. (20)-(22) and (26).
    Returns (A'_M, g_M, s_M).
    """
    x = [float(t) for t in x]
    V = np.asarray(V, dtype=np.float64)
    g, s = NEG_INF, 0.0
    A = np.zeros(V.shape[1])
    for xm, vm in zip(x, V):
        g_next = max(g, xm)
        if g_next == NEG_INF:
            continue  # only -inf so far: the state stays empty
        s_next = s * _exp(g - g_next) + _exp(xm - g_next)
        A = A * (s * _exp(g - g_next) / s_next) + (_exp(xm - g_next) / s_next) * vm
        g, s = g_next, s_next
    return A, g, s


def block_state(x_block, V_block):
    """(m, l, o) of one block of scores on its own: its max, its exponential sum
    and its normalised output.  A block whose scores are all -inf (fully
    masked) gives (-inf, 0, 0).
    Source: "从原始Softmax到在线Softmax" page, worked example 4 (per-block m, l, o)
    and the block quantities of the blocked recurrence.
    """
    x = [float(t) for t in x_block]
    V = np.asarray(V_block, dtype=np.float64)
    m = max(x)
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros(V.shape[1])
    e = [_exp(t - m) for t in x]
    l = sum(e)
    o = np.zeros(V.shape[1])
    for j, w in enumerate(e):
        o = o + (w / l) * V[j]
    return m, l, o


def merge_states(a, b):
    """Merge two (m, l, o-normalised) states over disjoint key sets.

    m = max(m_a, m_b); each side is rescaled by e^{m_side - m};
    l = e^{m_a-m} l_a + e^{m_b-m} l_b;
    o = (e^{m_a-m} l_a o_a + e^{m_b-m} l_b o_b) / l.
    An empty side (m = -inf) has weight 0.
    Source: "从原始Softmax到在线Softmax" page: the merge form of the blocked
    recurrence and its scale_old / scale_new update, worked example 4.
    """
    m_a, l_a, o_a = a
    m_b, l_b, o_b = b
    m = max(m_a, m_b)
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros_like(np.asarray(o_a, dtype=np.float64))
    sa, sb = _exp(m_a - m), _exp(m_b - m)
    l = sa * l_a + sb * l_b
    o = (sa * l_a * np.asarray(o_a) + sb * l_b * np.asarray(o_b)) / l
    return m, l, o


def blocked_attention(q, k, v, scale: float, causal: bool, Br: int, Bc: int):
    """Blocked recurrence with an unnormalised accumulator o~ (float64).

    For each query row i and each key block j+1:
      m_new  = max of the block's scores,
      m^{(j+1)} = max(m^{(j)}, m_new),
      l^{(j+1)} = e^{m^{(j)}-m^{(j+1)}} l^{(j)} + sum_k e^{s_k - m^{(j+1)}},
      o~^{(j+1)} = e^{m^{(j)}-m^{(j+1)}} o~^{(j)} + sum_k e^{s_k - m^{(j+1)}} v_k,
    and finally o = o~ / l, LSE = m + log l.  Starts from m = -inf, l = 0,
    o~ = 0; while the running max is still -inf (only masked keys seen) the
    state stays at its start.  Queries are grouped in blocks of Br rows (rows
    are independent, so Br only groups the work).
    Source: "从原始Softmax到在线Softmax" page, the online softmax derivation
    (m, l, o~ recurrences and o = o~/l) and LSE definition.

    q [B,H,N,d], k/v [B,H,M,d] -> (o [B,H,N,d], lse [B,H,N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    M = k.shape[2]
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N, Br):
                for i in range(i0, min(N, i0 + Br)):
                    m, l, ot = NEG_INF, 0.0, np.zeros(d)
                    for j0 in range(0, M, Bc):
                        js = range(j0, min(M, j0 + Bc))
                        s = []
                        for j in js:
                            if causal and j > i:
                                s.append(NEG_INF)
                            else:
                                s.append(scale * float(np.dot(q[b, h, i], k[b, h, j])))
                        m_new = max(s)
                        m_next = max(m, m_new)
                        if m_next == NEG_INF:
                            continue
                        alpha = _exp(m - m_next)
                        e = [_exp(t - m_next) for t in s]
                        l = alpha * l + sum(e)
                        acc = np.zeros(d)
                        for w, j in zip(e, js):
                            acc = acc + w * v[b, h, j]
                        ot = alpha * ot + acc
                        m = m_next
                    o[b, h, i] = ot / l
                    lse[b, h, i] = m + math.log(l)
    return o, lse


def split_merge_attention(q, k, v, scale: float, causal: bool, splits: int):
    """Attention by splitting the keys into ``splits`` contiguous ranges,
    computing each range's (m, l, o) with ``block_state`` and merging them
    left to right with ``merge_states``.  Returns (o, lse) like the others.
    Source: "从原始Softmax到在线Softmax" page, merge form and worked example 4.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    M = k.shape[2]
    bounds = [round(t * M / splits) for t in range(splits + 1)]
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                state = (NEG_INF, 0.0, np.zeros(d))
                for t in range(splits):
                    js = range(bounds[t], bounds[t + 1])
                    if len(js) == 0:
                        continue
                    x = [NEG_INF if (causal and j > i) else scale * float(np.dot(q[b, h, i], k[b, h, j]))
                         for j in js]
                    state = merge_states(state, block_state(x, v[b, h, bounds[t]:bounds[t + 1]]))
                m, l, ov = state
                o[b, h, i] = ov
                lse[b, h, i] = m + math.log(l)
    return o, lse
