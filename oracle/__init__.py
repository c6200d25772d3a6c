"""Float64 CPU oracle for the online-softmax attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this package.  It shares no code with the HIP
library (``online_softmax_10_amd``) and never imports it.

Two parts:

* ``liboracle.so`` (``oracle.c``): the plain definitions in float64 -- three-pass
  safe softmax, log-sum-exp, softmax cross-entropy, the one-pass normaliser
  recurrence, and exact attention softmax(mask(Q K^T scale)) V with its row LSE.
* ``recurrences`` (pure Python/numpy, small inputs only): the pages' other
  formulations -- the two-loop attention, the per-step normalised recurrence
  and the blocked (m, l, o~) recurrence with its merge form -- used only to
  cross-check the plain definition and to pin the pages' worked examples.

Every function takes and returns float64 numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out: str | None = None, src: str | None = None, extra_flags=()) -> str:
    """Compile the C oracle with gcc (float64, OpenMP).  Returns the .so path."""
    out = out or _LIB
    src = src or _SRC
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_softmax_f64.argtypes = [_f64p, _f64p, _i64, _i64]
    lib.oracle_logsumexp_f64.argtypes = [_f64p, _f64p, _i64, _i64]
    lib.oracle_xent_f64.argtypes = [_f64p, _i64p, _f64p, _f64p, _i64, _i64]
    lib.oracle_online_normalizer_f64.argtypes = [_f64p, _f64p, _f64p, _i64, _i64]
    lib.oracle_attn_rows_f64.argtypes = [_f64p, _f64p, _f64p, _i64, _i64, _i64, _i64, _i64,
                                         ctypes.c_double, ctypes.c_int, _i64p, _i64, _f64p, _f64p]
    lib.oracle_attn_masked_rows_f64.argtypes = [_f64p, _f64p, _f64p, _i64, _i64, _i64, _i64, _i64,
                                                ctypes.c_double, ctypes.c_int, _i64p, _f64p, _i64, _i64, _i64,
                                                _i64p, _i64, _f64p, _f64p]
    lib.oracle_attn_f64.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p, _i64, _i64, _i64, _i64, _i64,
                                    ctypes.c_double, ctypes.c_int]
    lib.oracle_num_threads.restype = ctypes.c_int
    for name in ("oracle_softmax_f64", "oracle_logsumexp_f64", "oracle_xent_f64", "oracle_online_normalizer_f64",
                 "oracle_attn_rows_f64", "oracle_attn_masked_rows_f64", "oracle_attn_f64"):
        getattr(lib, name).restype = None
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library.  ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(_f64p)


def _c64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def softmax(x, lib=None) -> np.ndarray:
    """Three-pass safe softmax over the last axis."""
    x = _c64(x)
    n = x.shape[-1]
    y = np.empty_like(x)
    (lib or load()).oracle_softmax_f64(_p(x), _p(y), x.size // n, n)
    return y


def logsumexp(x, lib=None) -> np.ndarray:
    x = _c64(x)
    n = x.shape[-1]
    out = np.empty(x.shape[:-1], dtype=np.float64)
    (lib or load()).oracle_logsumexp_f64(_p(x), _p(out), x.size // n, n)
    return out


def cross_entropy(x, labels, lib=None):
    """Per-row softmax cross-entropy, row LSE and their mean over rows.

    x [rows, n], labels [rows] integer class indices.  Returns (loss [rows],
    lse [rows], mean): loss_i = -log softmax(x_i)[labels_i] (NaN for a label
    outside [0, n)), mean = the page's batch mean of the losses (math.fsum).
    """
    import math

    x = _c64(x)
    n = x.shape[-1]
    rows = x.size // n
    lab = np.ascontiguousarray(np.asarray(labels, dtype=np.int64).reshape(rows))
    loss = np.empty(rows, dtype=np.float64)
    lse = np.empty(rows, dtype=np.float64)
    (lib or load()).oracle_xent_f64(_p(x), lab.ctypes.data_as(_i64p), _p(loss), _p(lse), rows, n)
    mean = math.fsum(loss.tolist()) / rows if rows else float("nan")
    return loss, lse, mean


def online_normalizer(x, lib=None):
    """(m_N, s_N) of the one-pass recurrence for each row of x."""
    x = _c64(x)
    n = x.shape[-1]
    m = np.empty(x.shape[:-1], dtype=np.float64)
    s = np.empty(x.shape[:-1], dtype=np.float64)
    (lib or load()).oracle_online_normalizer_f64(_p(x), _p(m), _p(s), x.size // n, n)
    return m, s


def attention(q, k, v, scale: float, causal, lib=None, kv_len=None, bias=None):
    """Exact attention.  q [B,H,N,d], k/v [B,H,M,d] float64 -> (o [B,H,N,d], lse [B,H,N]).

    causal, kv_len and bias as in attention_rows.
    """
    if causal not in (False, True) or kv_len is not None or bias is not None:
        q = _c64(q)
        B, H, N, d = q.shape
        o, lse = attention_rows(q, k, v, scale, causal, np.arange(B * H * N), lib, kv_len, bias)
        return o.reshape(B, H, N, d), lse.reshape(B, H, N)
    q, k, v = _c64(q), _c64(k), _c64(v)
    B, H, N, d = q.shape
    M = k.shape[2]
    assert k.shape == (B, H, M, d) and v.shape == (B, H, M, d) and M >= 1
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    (lib or load()).oracle_attn_f64(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, N, M, d,
                                    float(scale), int(bool(causal)))
    return o, lse


def attention_rows(q, k, v, scale: float, causal, rows, lib=None, kv_len=None, bias=None):
    """Exact attention for flat rows r=(b*H+h)*N+i -> (o [len(rows), d], lse [len(rows)]).

    causal: False / True (top-left: key j masked when j > i) / "bottom_right"
    (key j masked when j > i + M - N).  kv_len: optional [B] valid key counts
    (keys j >= kv_len[b] masked).  bias: optional additive score bias
    broadcastable to [B,H,N,M] (added after the scale; -inf masks a key).  A
    row with no visible key, or only -inf scores, gives o = 0, lse = -inf.
    """
    q, k, v = _c64(q), _c64(k), _c64(v)
    B, H, N, d = q.shape
    M = k.shape[2]
    assert k.shape == (B, H, M, d) and v.shape == (B, H, M, d) and M >= 1
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.ndim == 1 and (rows.size == 0 or (rows.min() >= 0 and rows.max() < B * H * N))
    mode = {False: 0, True: 1, "top_left": 1, "bottom_right": 2}[causal]
    kl = None
    if kv_len is not None:
        kl = np.ascontiguousarray(np.asarray(kv_len, dtype=np.int64).reshape(B))
    bp, bs = None, (0, 0, 0)
    if bias is not None:
        b64 = np.ascontiguousarray(bias, dtype=np.float64)
        bv = np.broadcast_to(b64, (B, H, N, M))
        assert bv.strides[3] == 8
        bp, bs = _p(b64), tuple(st // 8 for st in bv.strides[:3])
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    (lib or load()).oracle_attn_masked_rows_f64(_p(q), _p(k), _p(v), B, H, N, M, d, float(scale), mode,
                                                kl.ctypes.data_as(_i64p) if kl is not None else None,
                                                bp, *bs, rows.ctypes.data_as(_i64p), rows.size, _p(o), _p(lse))
    return o, lse
