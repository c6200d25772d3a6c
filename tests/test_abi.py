"""The C-ABI library loads without a GPU, exports every declared symbol, and
rejects invalid arguments with the documented codes before any HIP call
(these calls never touch a device; all pointers here are host addresses that
the library must not dereference)."""

import ctypes
import os
import re

import numpy as np
import pytest

import online_softmax_10_amd as osa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, HEADDIM, DTYPE, ALIGN, OVERFLOW, HIP, SCALE, SPLITS = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


def declared_functions():
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def L():
    return osa.lib()


@pytest.fixture(scope="module")
def buf():
    # 16-byte aligned host scratch; only its address is passed.
    raw = np.zeros(1024, dtype=np.uint8)
    base = raw.ctypes.data
    aligned = (base + 15) & ~15
    yield aligned
    del raw


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(osa.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(L, n), f"libattn.so does not export {n}"


def test_constants_match_header():
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    codes = dict((m[0], int(m[1])) for m in re.findall(r"(ATTN_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    for code, name in osa.ERROR_NAMES.items():
        assert codes[name] == code
    assert codes["ATTN_F32"] == osa.ATTN_F32 and codes["ATTN_BF16"] == osa.ATTN_BF16
    assert codes["ATTN_BF16_OUT_F32"] == osa.ATTN_BF16_OUT_F32
    assert int(re.search(r"#define ATTN_MAX_SPLITS (\d+)", text).group(1)) == osa.ATTN_MAX_SPLITS


def test_strerror(L):
    for code in list(osa.ERROR_NAMES) + [12345, -100]:
        s = L.attn_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert L.attn_strerror(0) == b"success"
    assert L.attn_last_error_detail() == b""


def call(L, buf, B=1, H=1, N=4, M=4, d=64, scale=0.125, causal=0, dtype=1, splits=0,
         q=None, k=None, v=None, o=None, lse=None):
    ptr = lambda p: buf if p is None else p
    return L.attn_fwd_splits(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, N, M, d, scale, causal, dtype,
                             splits, None)


def test_attn_validation(L, buf):
    assert call(L, buf, B=-1) == SHAPE
    assert call(L, buf, N=-3) == SHAPE
    assert call(L, buf, M=-1) == SHAPE
    assert call(L, buf, M=0) == SHAPE
    assert call(L, buf, dtype=3) == DTYPE
    assert call(L, buf, dtype=-1) == DTYPE
    for d in (0, 32, 96, 256):
        assert call(L, buf, d=d) == HEADDIM
    for s in (float("nan"), float("inf"), float("-inf")):
        assert call(L, buf, scale=s) == SCALE
    assert call(L, buf, splits=-1) == SPLITS
    assert call(L, buf, splits=osa.ATTN_MAX_SPLITS + 1) == SPLITS
    for name in ("q", "k", "v", "o", "lse"):
        assert call(L, buf, **{name: 0}) == NULL, name
        assert call(L, buf, **{name: buf + 4}) == ALIGN, name
        assert call(L, buf, **{name: buf + 8}) == ALIGN, name
    assert call(L, buf, N=2**31 // 64) == OVERFLOW
    assert call(L, buf, M=2**31 // 128, d=128) == OVERFLOW
    assert call(L, buf, B=2**31) == OVERFLOW
    assert call(L, buf, B=2**16, H=2**16) == OVERFLOW
    assert call(L, buf, B=2**13, H=2**10, N=512) == OVERFLOW  # 2^25 workgroups


def test_attn_empty_is_noop(L, buf):
    # B*H*N == 0 returns OK without touching the (null) pointers or a device.
    for kw in (dict(B=0), dict(H=0), dict(N=0)):
        assert call(L, buf, q=0, k=0, v=0, o=0, lse=0, **kw) == OK
    assert L.attn_fwd(None, None, None, None, None, 0, 1, 1, 1, 64, 1.0, 0, 1, None) == OK
    # validation of the other arguments still applies
    assert call(L, buf, N=0, d=32) == HEADDIM


def test_online_softmax_validation(L, buf):
    f = L.online_softmax
    assert f(buf, buf, -1, 3, None) == SHAPE
    assert f(buf, buf, 1, -3, None) == SHAPE
    assert f(buf, buf, 2, 0, None) == SHAPE
    assert f(None, buf, 1, 3, None) == NULL
    assert f(buf, None, 1, 3, None) == NULL
    assert f(buf + 4, buf, 1, 3, None) == ALIGN
    assert f(buf, buf + 8, 1, 3, None) == ALIGN
    assert f(buf, buf, 1, 2**31, None) == OVERFLOW
    assert f(buf, buf, 2**40, 2**30, None) == OVERFLOW
    assert f(None, None, 0, 5, None) == OK
    assert f(None, None, 0, 0, None) == OK


def test_online_softmax_lse_validation(L, buf):
    f = L.online_softmax_lse
    assert f(buf, buf, buf, -1, 3, None) == SHAPE
    assert f(buf, buf, buf, 2, 0, None) == SHAPE
    assert f(buf, None, None, 1, 3, None) == NULL   # no output at all
    assert f(None, buf, buf, 1, 3, None) == NULL
    assert f(buf, buf, buf + 2, 1, 3, None) == ALIGN  # lse needs 4-byte alignment
    assert f(buf, buf + 8, buf, 1, 3, None) == ALIGN
    assert f(buf, None, buf, 1, 2**31, None) == OVERFLOW
    assert f(None, None, None, 0, 5, None) == OK


def test_binding_raises_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 3)
    with pytest.raises(ValueError):
        osa.online_softmax(x)
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        osa.fwd(q, q, q)


def test_plan_kernel_choice():
    # Host-only query of the decomposition: the five workload shapes and the
    # regimes between them.
    assert osa.plan(2, 16, 4096, 4096, 128) == ("attn_fwd_bf16_w8_kernel", 1)
    assert osa.plan(1, 8, 16384, 16384, 128) == ("attn_fwd_bf16_w8_kernel", 1)
    assert osa.plan(2, 16, 4096, 4096, 64) == ("attn_fwd_bf16_w8_kernel", 1)
    assert osa.plan(2, 16, 4096, 4096, 128, dtype="bf16_out_f32") == ("attn_fwd_bf16_w8_kernel", 1)
    # 256 workgroups of 128 rows, one per CU: the keys split between two sets of waves
    assert osa.plan(4, 8, 1024, 1024, 64) == ("attn_fwd_bf16_kh_kernel", 1)
    # more than 256 workgroups of 128 rows, fewer than 256 of 256 rows: four waves
    assert osa.plan(1, 100, 384, 300, 64) == ("attn_fwd_bf16_kernel", 1)
    # fewer than 12 (d = 64) or 16 (d = 128) key tiles: four waves
    assert osa.plan(1, 2, 300, 960, 128) == ("attn_fwd_bf16_kernel", 1)
    assert osa.plan(1, 2, 300, 961, 128) == ("attn_fwd_bf16_kh_kernel", 1)
    assert osa.plan(4, 8, 1024, 704, 64) == ("attn_fwd_bf16_kernel", 1)
    assert osa.plan(4, 8, 1024, 705, 64) == ("attn_fwd_bf16_kh_kernel", 1)
    assert osa.plan(4, 8, 1024, 1024, 64, dtype="bf16_out_f32") == ("attn_fwd_bf16_kh_kernel", 1)
    name, s = osa.plan(32, 32, 1, 8192, 128)
    assert name == "attn_decode_kernel" and 1 <= s <= osa.ATTN_MAX_SPLITS
    # the fp32 workload: one launch, keys split among the waves of each 16-row workgroup
    assert osa.plan(1, 1, 256, 256, 64, "f32") == ("attn_fwd_f32_small_kernel", 1)
    assert osa.plan(1, 1, 256, 256, 64, "f32", num_splits=1) == ("attn_fwd_f32_kernel", 1)
    assert osa.plan(1, 1, 100, 5000, 64, "f32")[0] == "attn_fwd_f32_kernel"  # long key ranges: split partials
    assert osa.plan(1, 1, 256, 256, 128, "f32") == ("attn_fwd_f32_small_kernel", 1)
    assert osa.plan(1, 1, 256, 1025, 128, "f32")[0] == "attn_fwd_f32_kernel"
    # Few query tiles and a long key range: split partials, merged afterwards.
    name, s = osa.plan(1, 1, 100, 8000, 64)
    assert name == "attn_fwd_bf16_kernel" and s > 1
    name, s = osa.plan(1, 1, 4096, 4096, 128)
    assert name == "attn_fwd_bf16_kernel" and s > 1
    # Few query tiles but a short key loop: the split's workspace, merge kernel
    # and host calls would cost more than they save.
    assert osa.plan(2, 4, 512, 512, 64) == ("attn_fwd_bf16_kernel", 1)
    assert osa.plan(1, 16, 1024, 1024, 128) == ("attn_fwd_bf16_kh_kernel", 1)
    assert osa.plan(1, 2, 2048, 2048, 64) == ("attn_fwd_bf16_kh_kernel", 1)
    assert osa.plan(1, 1, 256, 256, 64, "f32", num_splits=2) == ("attn_fwd_f32_kernel", 2)
    # An explicit single pass on a small problem splits its keys between two
    # sets of waves of each workgroup (no partials, no merge kernel); the
    # eight-wave kernel never writes partials.
    assert osa.plan(1, 1, 100, 5000, 64, num_splits=1) == ("attn_fwd_bf16_kh_kernel", 1)
    assert osa.plan(2, 16, 4096, 4096, 128, num_splits=4) == ("attn_fwd_bf16_kernel", 4)
    assert osa.plan(1, 1, 4, 8192, 128, num_splits=8) == ("attn_decode_kernel", 8)


def test_plan_rejects_like_attn_fwd(L):
    splits = ctypes.c_int(7)
    for args in ((0, 1, 4, 4, 64, 1, 0), (1, 1, 0, 4, 64, 1, 0), (1, 1, 4, 0, 64, 1, 0), (1, 1, 4, 4, 96, 1, 0),
                 (1, 1, 4, 4, 64, 3, 0), (1, 1, 4, 4, 64, 1, -1), (1, 1, 4, 4, 64, 1, osa.ATTN_MAX_SPLITS + 1),
                 (1, 1, 2**31 // 64, 4, 64, 1, 0)):
        splits.value = 7
        assert L.attn_fwd_plan(*args, ctypes.byref(splits)) is None, args
        assert splits.value == 0
    assert L.attn_fwd_plan(1, 1, 4, 4, 64, 1, 0, None) is not None


def test_softmax_xent_validation(L, buf):
    f = L.softmax_xent
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    assert f(buf, buf, buf, buf, buf, -1, 3, None) == SHAPE
    assert f(buf, buf, buf, buf, buf, 2, -1, None) == SHAPE
    assert f(buf, buf, buf, buf, buf, 2, 0, None) == SHAPE
    assert f(None, buf, buf, None, None, 2, 3, None) == NULL
    assert f(buf, None, buf, None, None, 2, 3, None) == NULL
    assert f(buf, buf, None, None, None, 2, 3, None) == NULL
    assert f(buf + 4, buf, buf, None, None, 2, 3, None) == ALIGN
    assert f(buf, buf + 4, buf, None, None, 2, 3, None) == ALIGN
    assert f(buf, buf, buf + 2, None, None, 2, 3, None) == ALIGN
    assert f(buf, buf, buf, buf + 1, None, 2, 3, None) == ALIGN
    assert f(buf, buf, buf, None, buf + 3, 2, 3, None) == ALIGN
    assert f(buf, buf, buf, None, None, 1, 2**31, None) == OVERFLOW
    assert f(buf, buf, buf, None, None, 2**40, 2**30, None) == OVERFLOW
    assert f(None, None, None, None, None, 0, 5, None) == OK
    assert f(None, None, None, None, None, 0, 0, None) == OK


def test_bias_validation(L, buf):
    f = L.attn_fwd_masked
    args = lambda mask: (buf, buf, buf, buf, buf, 1, 1, 4, 4, 64, 0.125, ctypes.byref(mask), 1, 0, None)
    assert f(*args(osa.AttnMask(0, None, buf + 4, 0, 0, 4))) == ALIGN  # bias pointer not 16-byte aligned
    assert f(*args(osa.AttnMask(0, None, buf, 0, 0, 6))) == ALIGN      # row stride not a multiple of 4
    assert f(*args(osa.AttnMask(0, None, buf, 2, 0, 4))) == ALIGN      # batch stride not a multiple of 4
    assert f(*args(osa.AttnMask(0, None, buf, 0, -4, 4))) == SHAPE     # negative stride
    assert f(*args(osa.AttnMask(1, buf + 2, buf, 0, 0, 4))) == ALIGN   # kv_len checked too
    # A bias spanning 4 GiB or more from its base (32-bit offsets in the kernels).
    big = lambda sb: (buf, buf, buf, buf, buf, 2, 1, 4, 4, 64, 0.125,
                      ctypes.byref(osa.AttnMask(0, None, buf, sb, 0, 4)), 1, 0, None)
    assert f(*big(2**30)) == OVERFLOW


def test_noalloc_validation(L, buf):
    # attn_fwd_masked_noalloc validates like attn_fwd_masked and rejects a split
    # workspace beyond its static scratch, all before any HIP call.
    f = L.attn_fwd_masked_noalloc
    args = lambda mask, **kw: (buf, buf, buf, buf, buf, kw.get("B", 1), kw.get("H", 1), kw.get("N", 4),
                               kw.get("M", 4), kw.get("d", 64), 0.125, mask, 1, kw.get("splits", 0), None)
    assert f(*args(ctypes.byref(osa.AttnMask(3, None)))) == -10
    assert f(*args(None, B=0)) == OK
    assert f(*args(None, splits=-1)) == SPLITS
    assert f(*args(None, d=96)) == HEADDIM
    # 256 splits x 300 rows x (128 + 1) floats = 39.6 MB > 32 MiB
    assert f(*args(None, N=300, M=300000, d=128, splits=256)) == -11  # ATTN_ERR_WORKSPACE
    assert 256 * 300 * 129 * 4 > osa.NOALLOC_SCRATCH_BYTES
    with open(HEADER, encoding="utf-8") as h:
        assert int(re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES (\d+)", h.read()).group(1)) == osa.NOALLOC_SCRATCH_BYTES


def test_masked_validation(L, buf):
    f = L.attn_fwd_masked
    m = osa.AttnMask(3, None)
    args = lambda mask, **kw: (buf, buf, buf, buf, buf, kw.get("B", 1), 1, 4, 4, 64, 0.125, mask, 1,
                               kw.get("splits", 0), None)
    assert f(*args(ctypes.byref(m))) == -10  # ATTN_ERR_MASK
    m = osa.AttnMask(-1, None)
    assert f(*args(ctypes.byref(m))) == -10
    m = osa.AttnMask(2, buf + 2)
    assert f(*args(ctypes.byref(m))) == ALIGN
    m = osa.AttnMask(1, None)
    assert f(*args(ctypes.byref(m), B=0)) == OK
    assert f(*args(None, B=0)) == OK
    assert f(*args(ctypes.byref(m), splits=-1)) == SPLITS
