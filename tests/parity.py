"""Helpers for comparing the HIP path (through the C ABI) with the oracle.

Tolerances (max-abs, element by element, as the workloads state them):
  * bf16 inputs: |lse - lse_ref| <= 5e-3, and
        |o - o_ref| <= 1e-2 + ulp_bf16(o_ref) / 2,
    i.e. 1e-2 for the computation plus the unavoidable rounding of the stored
    bf16 output (rounding the exact float64 output itself to bf16 already
    moves it by up to half a bf16 ulp, 0.0156 for |o| in [4, 8)).
  * fp32 inputs: |o - o_ref| <= 1e-5 and |lse - lse_ref| <= 1e-5 on the fp32
    workload (literal); elsewhere the larger of 1e-5 and the rounding bound
    of f32_bounds, per element, derived from the fp32 arithmetic the kernels
    do (it exceeds 1e-5 only where the scores or the key count are large).
The raw max-abs errors are reported alongside.
"""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle
import seeded_inputs as si

F32_TOL = 1e-5
BF16_O_TOL = 1e-2
BF16_LSE_TOL = 5e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    h = np.exp2(e - 8.0)
    return np.where(a > 0, h, 2.0 ** -134)


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def gpu_attention(q, k, v, dtype: str, scale: float, causal: bool, splits: int = 0):
    """Run the HIP path; returns (o float64 [B,H,N,d], lse float64 [B,H,N]) on the host."""
    import torch

    import online_softmax_10_amd as osa

    qd, kd, vd = (to_device(a, dtype) for a in (q, k, v))
    o, lse = osa.fwd_splits(qd, kd, vd, scale=scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


U = 2.0 ** -24           # unit roundoff of fp32
EPS_EXP = 2.0 ** -22     # relative error allowed for the hardware exp2 (v_exp_f32)
LAMBDA = 6.0             # confidence factor of the probabilistic sum bound


def f32_bounds(q, k, v, scale, causal=False, kv_len=None, bias=None):
    """Per-element error bounds (o [B,H,N,d], lse [B,H,N]) for the fp32 path.

    q [B,H,N,d], k, v [B,H,M,d] float64 (the stored fp32 values).  The kernels
    compute, per query row and visible key j:
      s_j = scale <q, k_j>      an fp32 dot product of length d (MFMA), error
                                <= gamma_d sum_k |q_k k_jk|, gamma_d = d u / (1 - d u);
      x_j = c s_j - m           one FMA (c = |scale| log2 e rounded), relative
                                error u of x_j plus 2u of s_j from c;
      p_j = 2^{x_j}             relative error <= EPS_EXP;
    and where the keys of a row are shared out (over the waves of a workgroup
    or over split workgroups), each part's state is weighted by one more
    2^{m_part - M} and a division by L when the parts are merged: EPS_EXP + 2u.
    So ln p_j is off by at most
      E_j = |scale| gamma_d A_j + 2u |s_j| + u (m - s_j) + 2 EPS_EXP + 2u
    (natural units, A_j = sum_k |q_k k_jk|).  To first order, perturbing each
    log-weight by at most E_j moves o = sum_j w_j v_j by at most
      sum_j w_j E_j |v_j - o|  <=  (w E) |v| + |o| sum_j w_j E_j
    and LSE = m + log sum_j e^{s_j - m} by at most sum_j w_j E_j.  The sums over
    the keys (l, and o~ = sum_j p_j v_j, each rescaled once per 32-key tile)
    are fp32 sums of M' = M + 2 ceil(M/32) terms; their error is bounded with
    the probabilistic model of rounding (independent zero-mean errors,
    Higham and Mary 2019): LAMBDA sqrt(M') u times the sum of the magnitudes
    (the worst case M' u is vacuous for M near 10^5).  The final division and
    the LSE's own rounding add u |o| and 2u |lse|.  Returns (bound_o,
    bound_lse), each at least 1e-5.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    M = k.shape[2]
    kt = np.swapaxes(k, -1, -2)
    s = float(scale) * np.matmul(q, kt)
    A = np.matmul(np.abs(q), np.abs(kt))
    i = np.arange(N)[:, None]
    j = np.arange(M)[None, :]
    vis = np.ones((B, 1, N, M), dtype=bool)
    if causal in (True, "top_left"):
        vis = vis & (j <= i)[None, None]
    elif causal == "bottom_right":
        vis = vis & (j <= i + (M - N))[None, None]
    if kv_len is not None:
        kl = np.clip(np.asarray(kv_len), 0, M).reshape(B, 1, 1, 1)
        vis = vis & (j[None, None] < kl)
    if bias is not None:
        s = s + np.broadcast_to(np.asarray(bias, dtype=np.float64), s.shape)
    vis = np.broadcast_to(vis, s.shape) & np.isfinite(s)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(vis, np.exp(s - m), 0.0)
    lsum = w.sum(axis=-1, keepdims=True)
    w = w / np.where(lsum > 0, lsum, 1.0)
    gd = d * U / (1.0 - d * U)
    sv = np.where(vis, s, 0.0)
    E = np.where(vis, abs(float(scale)) * gd * A + 2 * U * np.abs(sv) + U * (m - sv) + 2 * EPS_EXP + 2 * U, 0.0)
    wE = w * E
    o = np.matmul(w, v)
    sum_wE = wE.sum(axis=-1)
    mp = M + 2 * ((M + 31) // 32)
    gsum = LAMBDA * np.sqrt(mp) * U
    lse = np.where(lsum[..., 0] > 0, m[..., 0] + np.log(np.where(lsum[..., 0] > 0, lsum[..., 0], 1.0)), 0.0)
    bo = np.matmul(wE, np.abs(v)) + np.abs(o) * sum_wE[..., None] + gsum * (np.matmul(w, np.abs(v)) + np.abs(o)) \
        + U * np.abs(o)
    bl = sum_wE + gsum + 2 * U * np.abs(lse)
    return np.maximum(F32_TOL, bo), np.maximum(F32_TOL, bl)


def compare(o, lse, o_ref, lse_ref, dtype: str, what: str, bounds=None) -> dict:
    """Assert the tolerance rule; return the measured errors.

    bounds: for fp32 inputs, (bound_o, bound_lse) arrays shaped like o and
    lse (f32_bounds); None applies the literal 1e-5.
    """
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err_o = np.abs(o - o_ref)
    err_l = np.abs(np.asarray(lse, dtype=np.float64) - np.asarray(lse_ref, dtype=np.float64))
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    if dtype == "bf16":
        bound = BF16_O_TOL + half_ulp_bf16(o_ref)
        lse_tol = BF16_LSE_TOL
    elif bounds is None:
        bound = np.full_like(o_ref, F32_TOL)
        lse_tol = F32_TOL
    else:
        bound = np.asarray(bounds[0], dtype=np.float64)
        lse_tol = np.asarray(bounds[1], dtype=np.float64)
    stats = {"max_abs_o": float(err_o.max(initial=0.0)), "max_abs_lse": float(err_l.max(initial=0.0)),
             "worst_o_over_bound": float((err_o / bound).max(initial=0.0))}
    log(f"  {what}: max|do|={stats['max_abs_o']:.3e} max|dlse|={stats['max_abs_lse']:.3e} "
        f"worst do/bound={stats['worst_o_over_bound']:.3f}")
    bad = np.argwhere(err_o > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} output elements out of tolerance; first at {tuple(bad[0])}: "
                           f"got {o[tuple(bad[0])]}, want {o_ref[tuple(bad[0])]}")
    badl = np.argwhere(err_l > lse_tol)
    assert badl.size == 0, (f"{what}: {len(badl)} lse values out of tolerance; first at {tuple(badl[0])}: "
                            f"got {np.asarray(lse)[tuple(badl[0])]}, want {np.asarray(lse_ref)[tuple(badl[0])]}")
    return stats


def check_full(w: si.Workload, seed: int, splits: int = 0, qkv=None, f32_literal: bool = False) -> dict:
    """Whole-output parity for a workload small enough for the full oracle.

    fp32: the derived bound of f32_bounds (at least 1e-5), or with
    f32_literal the workload's 1e-5 as stated."""
    q, k, v = qkv if qkv is not None else si.make_qkv(w, seed)
    log(f"[gpu] {w.name} B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} causal={w.causal} "
        f"seed={seed} splits={splits}")
    o, lse = gpu_attention(q, k, v, w.dtype, w.scale, w.causal, splits)
    qf, kf, vf = (si.to_f64(a, w.dtype) for a in (q, k, v))
    o_ref, lse_ref = oracle.attention(qf, kf, vf, w.scale, w.causal)
    bounds = None
    if w.dtype != "bf16" and not f32_literal:
        bounds = f32_bounds(qf, kf, vf, w.scale, w.causal)
    return compare(o, lse, o_ref, lse_ref, w.dtype, f"{w.name} seed={seed} splits={splits}", bounds)


def check_sampled(w: si.Workload, seed: int, count: int, splits: int = 0) -> dict:
    """Full-size run, oracle on sampled rows."""
    q, k, v = si.make_qkv(w, seed)
    log(f"[gpu] {w.name} full size B={w.B} H={w.H} N={w.N} M={w.M} d={w.d} {w.dtype} causal={w.causal} "
        f"seed={seed} splits={splits}, {count} sampled rows")
    o, lse = gpu_attention(q, k, v, w.dtype, w.scale, w.causal, splits)
    rows = si.sample_rows(w, count)
    o_ref, lse_ref = oracle.attention_rows(si.to_f64(q, w.dtype), si.to_f64(k, w.dtype), si.to_f64(v, w.dtype),
                                           w.scale, w.causal, rows)
    assert w.dtype == "bf16", "sampled checks are for bf16 workloads"
    return compare(o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, w.dtype,
                   f"{w.name} seed={seed} sampled")
