"""Python binding of libattn.so: the MI355X online-softmax attention forward.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``; torch provides device
memory and the stream.  There is no CPU or torch fallback: if the library is
missing or a call fails, an exception is raised.

    o, lse = fwd(q, k, v, scale=None, causal=False)      # q [B,H,N,d], k/v [B,H,M,d]
    y = online_softmax(x)                                  # x [rows, n] float32
    loss, lse, mean = softmax_xent(x, labels)              # labels [rows] int64
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "fwd_splits", "fwd_noalloc", "fwd_kv_outer", "NOALLOC_SCRATCH_BYTES", "online_softmax", "logsumexp", "softmax_xent", "plan", "lib", "AttnMask", "CAUSAL_MODES", "LIB_PATH", "AttnError",
           "ATTN_F32", "ATTN_BF16", "ATTN_BF16_OUT_F32", "ATTN_MAX_SPLITS", "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_BF16_OUT_F32 = 2
ATTN_MAX_SPLITS = 256
NOALLOC_SCRATCH_BYTES = 33554432  # ATTN_NOALLOC_SCRATCH_BYTES
ERROR_NAMES = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_HEADDIM",
               -4: "ATTN_ERR_DTYPE", -5: "ATTN_ERR_ALIGN", -6: "ATTN_ERR_OVERFLOW", -7: "ATTN_ERR_HIP",
               -8: "ATTN_ERR_SCALE", -9: "ATTN_ERR_SPLITS", -10: "ATTN_ERR_MASK", -11: "ATTN_ERR_WORKSPACE"}
EXPORTED_SYMBOLS = ("attn_fwd", "attn_fwd_splits", "attn_fwd_masked", "attn_fwd_masked_noalloc", "attn_fwd_kv_outer",
                    "online_softmax",
                    "online_softmax_lse", "softmax_xent", "attn_fwd_plan", "attn_strerror", "attn_last_error_detail")

# attn_causal of include/attn.h, by the names fwd() accepts.
CAUSAL_MODES = {False: 0, True: 1, "none": 0, "top_left": 1, "bottom_right": 2}


class AttnMask(ctypes.Structure):
    """struct attn_mask of include/attn.h."""
    _fields_ = [("causal", ctypes.c_int), ("kv_len", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("bias_stride_b", ctypes.c_int64), ("bias_stride_h", ctypes.c_int64),
                ("bias_stride_n", ctypes.c_int64)]

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        detail = ""
        if _lib is not None:
            detail = _lib.attn_strerror(code).decode()
            if code == -7:
                detail += f" [{_lib.attn_last_error_detail().decode()}]"
        super().__init__(f"{where}: {ERROR_NAMES.get(code, code)}: {detail}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded C library (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m online_softmax_10_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                               ctypes.c_int, ctypes.c_int, vp]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_fwd_splits.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.attn_fwd_splits.restype = ctypes.c_int
        L.attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                      ctypes.POINTER(AttnMask), ctypes.c_int, ctypes.c_int, vp]
        L.attn_fwd_masked.restype = ctypes.c_int
        L.attn_fwd_masked_noalloc.argtypes = L.attn_fwd_masked.argtypes
        L.attn_fwd_masked_noalloc.restype = ctypes.c_int
        L.attn_fwd_kv_outer.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_int, ctypes.c_int, vp]
        L.attn_fwd_kv_outer.restype = ctypes.c_int
        L.online_softmax.argtypes = [vp, vp, i64, i64, vp]
        L.online_softmax.restype = ctypes.c_int
        L.online_softmax_lse.argtypes = [vp, vp, vp, i64, i64, vp]
        L.online_softmax_lse.restype = ctypes.c_int
        L.attn_strerror.argtypes = [ctypes.c_int]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_last_error_detail.argtypes = []
        L.attn_last_error_detail.restype = ctypes.c_char_p
        L.softmax_xent.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp]
        L.softmax_xent.restype = ctypes.c_int
        L.attn_fwd_plan.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_int)]
        L.attn_fwd_plan.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _stream_handle(device):
    """The raw HIP stream of torch's current stream on ``device``."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return ctypes.c_void_p(raw(device.index if device.index is not None else torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected torch.bfloat16 or torch.float32")


def _check_output(name, t, shape, dtype, device):
    if tuple(t.shape) != shape or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {device}; "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _bias_operand(bias, B, H, N, M, device):
    """A float32 bias broadcastable to [B,H,N,M] -> (tensor to pass, (sb, sh, sn)).

    The library reads rows of M contiguous floats at 16-byte aligned addresses;
    a bias that is not laid out so is copied into rows padded to a multiple of
    4 elements (broadcast dimensions stay unexpanded).
    """
    import torch

    if bias.dtype != torch.float32 or bias.device != device:
        raise ValueError(f"bias must be a float32 tensor on {device}")
    if bias.dim() > 4:
        raise ValueError("bias must have at most 4 dimensions [B,H,N,M]")
    try:
        view = bias.expand(B, H, N, M)
    except RuntimeError as e:
        raise ValueError(f"bias of shape {tuple(bias.shape)} does not broadcast to {(B, H, N, M)}") from e
    st = view.stride()
    if st[3] != 1 or any(s % 4 for s in st[:3]) or view.data_ptr() % 16:
        src = bias.reshape((1,) * (4 - bias.dim()) + tuple(bias.shape))
        lead = src.shape[:3]
        padded = torch.empty(lead + ((M + 3) // 4 * 4,), dtype=torch.float32, device=device)
        padded[..., :M].copy_(src.expand(lead + (M,)))
        view = padded[..., :M].expand(B, H, N, M)
        st = view.stride()
    return view, st[:3]


def fwd_noalloc(q, k, v, scale=None, causal=False, num_splits=0, out=None, lse=None, kv_len=None, bias=None,
                out_dtype=None):
    """fwd_splits through attn_fwd_masked_noalloc: the split workspace is the
    library's static device scratch (NOALLOC_SCRATCH_BYTES per GPU) instead of
    a stream-ordered allocation.  Pass out and lse to allocate nothing at all.
    Calls that overlap on one GPU race on the scratch."""
    return fwd_splits(q, k, v, scale=scale, causal=causal, num_splits=num_splits, out=out, lse=lse, kv_len=kv_len,
                      bias=bias, out_dtype=out_dtype, _noalloc=True)


def fwd_splits(q, k, v, scale=None, causal=False, num_splits=0, out=None, lse=None, kv_len=None, bias=None,
               out_dtype=None, _noalloc=False):
    """Attention forward with an explicit split count (0 = library's choice).

    q [B,H,N,d], k and v [B,H,M,d]: contiguous CUDA/HIP tensors of one dtype
    (bfloat16 or float32).  causal: False, True / "top_left" (key j masked for
    query i when j > i) or "bottom_right" (when j > i + M - N).  kv_len:
    optional contiguous int32 GPU tensor [B] of valid key counts (keys j >=
    kv_len[b] masked).  bias: optional float32 GPU tensor broadcastable to
    [B,H,N,M], added to the scaled scores (-inf masks a key).  out_dtype:
    torch.float32 with bfloat16 inputs writes o in float32 (the same
    arithmetic, o not rounded to bf16); default: the inputs' dtype.  Returns
    (o [B,H,N,d], lse [B,H,N] float32); a row with no visible key (or only
    -inf scores) gets o = 0, lse = -inf.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B,H,rows,d]")
    B, H, N, d = q.shape
    M = k.shape[2]
    if tuple(k.shape) != (B, H, M, d) or tuple(v.shape) != (B, H, M, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    code = _dtype_code(q)
    o_dtype = q.dtype if out_dtype is None else out_dtype
    if o_dtype != q.dtype:
        if q.dtype != torch.bfloat16 or o_dtype != torch.float32:
            raise ValueError("out_dtype other than the inputs' is only float32 with bfloat16 inputs")
        code = ATTN_BF16_OUT_F32
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    else:
        _check_output("out", out, (B, H, N, d), o_dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_output("lse", lse, (B, H, N), torch.float32, q.device)
    if causal not in CAUSAL_MODES:
        raise ValueError(f"causal must be one of {sorted(map(str, CAUSAL_MODES))}, got {causal!r}")
    mode = CAUSAL_MODES[causal]
    if kv_len is None and mode != 2 and bias is None and not _noalloc:
        rc = lib().attn_fwd_splits(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   B, H, N, M, d, float(scale), mode, code, int(num_splits),
                                   _stream_handle(q.device))
        if rc != 0:
            raise AttnError(rc, "attn_fwd_splits")
        return out, lse
    if kv_len is not None:
        if (kv_len.dtype != torch.int32 or kv_len.device != q.device or not kv_len.is_contiguous()
                or kv_len.numel() != B):
            raise ValueError(f"kv_len must be a contiguous int32 tensor of {B} entries on {q.device}")
    mask = AttnMask(mode, kv_len.data_ptr() if kv_len is not None else None)
    if bias is not None:
        bias, (sb, sh, sn) = _bias_operand(bias, B, H, N, M, q.device)
        mask.bias, mask.bias_stride_b, mask.bias_stride_h, mask.bias_stride_n = bias.data_ptr(), sb, sh, sn
    entry = lib().attn_fwd_masked_noalloc if _noalloc else lib().attn_fwd_masked
    rc = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
               B, H, N, M, d, float(scale), ctypes.byref(mask), code, int(num_splits), _stream_handle(q.device))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_masked_noalloc" if _noalloc else "attn_fwd_masked")
    return out, lse


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, kv_len=None, bias=None, out_dtype=None):
    """softmax(mask(q k^T * scale + bias)) v and the row log-sum-exp (natural log).

    causal, kv_len, bias and out_dtype as in fwd_splits.
    """
    return fwd_splits(q, k, v, scale=scale, causal=causal, num_splits=0, out=out, lse=lse, kv_len=kv_len,
                      bias=bias, out_dtype=out_dtype)


def fwd_kv_outer(q, k, v, scale=None, causal=False, out=None, lse=None):
    """The same attention in the key/value-outer loop order (row state through
    HBM after every 64-key block); bf16 only.  For measuring loop orders."""
    import torch

    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("fwd_kv_outer takes bfloat16 q, k, v")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B,H,rows,d]")
    B, H, N, d = q.shape
    M = k.shape[2]
    if tuple(k.shape) != (B, H, M, d) or tuple(v.shape) != (B, H, M, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous GPU tensor on q's device")
    if causal not in (False, True):
        raise ValueError("fwd_kv_outer supports causal=False or True (top-left)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    else:
        _check_output("out", out, (B, H, N, d), q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_output("lse", lse, (B, H, N), torch.float32, q.device)
    rc = lib().attn_fwd_kv_outer(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 B, H, N, M, d, float(scale), int(bool(causal)), ATTN_BF16,
                                 _stream_handle(q.device))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_kv_outer")
    return out, lse


def plan(B, H, N, M, d, dtype="bf16", num_splits=0):
    """(kernel name, split count) that fwd_splits would use for these sizes.

    Host-side query of the library's work decomposition; launches nothing.
    Raises ValueError for sizes the library rejects or with nothing to compute.
    """
    code = {"bf16": ATTN_BF16, "f32": ATTN_F32, "bf16_out_f32": ATTN_BF16_OUT_F32}[dtype]
    splits = ctypes.c_int(0)
    name = lib().attn_fwd_plan(B, H, N, M, d, code, num_splits, ctypes.byref(splits))
    if name is None:
        raise ValueError(f"no plan for B={B} H={H} N={N} M={M} d={d} {dtype} num_splits={num_splits}")
    return name.decode(), splits.value


def online_softmax(x, out=None, return_lse=False, lse=None):
    """Row-wise softmax of a contiguous float32 GPU tensor over its last axis.

    return_lse: also return the rows' log-sum-exp (float32, x.shape[:-1]),
    i.e. (y, lse).
    """
    import torch

    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    n = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // n if n > 0 else 0
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_output("out", out, tuple(x.shape), torch.float32, x.device)
    if not return_lse:
        rc = lib().online_softmax(x.data_ptr(), out.data_ptr(), rows, n, _stream_handle(x.device))
        if rc != 0:
            raise AttnError(rc, "online_softmax")
        return out
    lse = _lse_output(x, lse)
    rc = lib().online_softmax_lse(x.data_ptr(), out.data_ptr(), lse.data_ptr(), rows, n, _stream_handle(x.device))
    if rc != 0:
        raise AttnError(rc, "online_softmax_lse")
    return out, lse


def _lse_output(x, lse):
    import torch

    shape = tuple(x.shape[:-1]) if x.dim() > 0 else ()
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_output("lse", lse, shape, torch.float32, x.device)
    return lse


def logsumexp(x, out=None):
    """log sum exp over the last axis of a contiguous float32 GPU tensor: the
    normaliser of online_softmax alone, one read of x."""
    import torch

    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    n = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // n if n > 0 else 0
    out = _lse_output(x, out)
    rc = lib().online_softmax_lse(x.data_ptr(), None, out.data_ptr(), rows, n, _stream_handle(x.device))
    if rc != 0:
        raise AttnError(rc, "online_softmax_lse")
    return out


def softmax_xent(x, labels, out=None, lse=None, mean=True):
    """Per-row softmax cross-entropy against integer labels.

    x: contiguous float32 GPU tensor, softmax over its last axis (rows = the
    product of the other axes); labels: contiguous int64 GPU tensor with one
    label per row.  Returns (loss [rows] float32, lse [rows] float32, mean: a
    one-element float32 tensor, or None when mean=False).  A label outside
    [0, n) gives a NaN loss for its row.
    """
    import torch

    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous float32 GPU tensor with at least one axis")
    n = x.shape[-1]
    rows = x.numel() // n if n > 0 else 0
    if labels.dtype != torch.int64 or not labels.is_contiguous() or labels.device != x.device:
        raise ValueError("labels must be a contiguous int64 tensor on x's device")
    if labels.numel() != rows:
        raise ValueError(f"labels has {labels.numel()} entries for {rows} rows")
    if out is None:
        out = torch.empty((rows,), dtype=torch.float32, device=x.device)
    else:
        _check_output("out", out, (rows,), torch.float32, x.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=x.device)
    else:
        _check_output("lse", lse, (rows,), torch.float32, x.device)
    m = torch.empty((1,), dtype=torch.float32, device=x.device) if mean else None
    rc = lib().softmax_xent(x.data_ptr(), labels.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            m.data_ptr() if m is not None else None, rows, n, _stream_handle(x.device))
    if rc != 0:
        raise AttnError(rc, "softmax_xent")
    return out, lse, m
