"""GPU parity of attn_fwd (through the C ABI) against the float64 oracle.

Every case prints its name, shape and seed before it touches the GPU.
"""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import check_full, compare, f32_bounds, gpu_attention, log

pytestmark = pytest.mark.gpu

W = si.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_10_amd as osa

    osa.lib()  # fail loudly if the HIP library is missing
    yield


# ------------------------------------------------------------------ the workloads

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_c1_fp32_full(seed):
    # the fp32 workload keeps the literal 1e-5
    check_full(W["c1"], seed, f32_literal=True)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_c2_bf16_full(seed):
    check_full(W["c2"], seed)


@pytest.mark.parametrize("seed", [0, 1])
def test_c3_causal_full(seed):
    # every one of the 131072 output rows against the oracle
    check_full(W["c3"], seed)


def test_c3_causal_reduced_full():
    # c3's distributions and causal mask with fewer heads, every output row checked
    check_full(W["c3"].with_shape(B=1, H=2, N=2048, M=2048), 0)


def test_c4_long_causal_full():
    # every one of the 131072 output rows (16384 keys each, peaked rows that
    # move the lazy shift) against the oracle
    check_full(W["c4"], 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_c5_decode_full(seed):
    check_full(W["c5"], seed)


def test_c5_decode_reduced_full():
    check_full(W["c5"].with_shape(B=2, H=4), 0)


# ------------------------------------------------------------------ tiles and ragged tails

SIZES = [1, 3, 127, 129, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_shapes(dtype, d, causal):
    base = si.Workload("ragged", 1, 2, 1, 1, d, dtype, causal, "normal")
    for i, N in enumerate(SIZES):
        for j, M in enumerate(SIZES):
            if (i + j) % 2:  # a checkerboard of the grid keeps the case count modest
                continue
            check_full(base.with_shape(N=N, M=M), seed=100 + 10 * i + j)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_n_greater_than_m_causal(dtype):
    # causal with more queries than keys: rows past M see every key
    check_full(si.Workload("tall", 2, 1, 300, 70, 64, dtype, True, "normal"), 5)


# ------------------------------------------------------------------ split invariance

@pytest.mark.parametrize("splits", [1, 2, 7, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_forced_splits_match_oracle(splits, causal):
    w = si.Workload("split", 2, 3, 200, 1000, 128, "bf16", causal, "normal")
    check_full(w, 7, splits=splits)


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_forced_splits_fp32(splits):
    w = si.Workload("split32", 1, 2, 130, 700, 64, "f32", False, "uniform01")
    check_full(w, 8, splits=splits)


@pytest.mark.parametrize("N", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_path(N, dtype, causal):
    w = si.Workload("decode", 3, 5, N, 777, 128 if dtype == "bf16" else 64, dtype, causal, "normal")
    check_full(w, 11 + N)
    check_full(w, 11 + N, splits=5)


def test_split_paths_agree_on_c2():
    w = W["c2"]
    q, k, v = si.make_qkv(w, 0)
    log("[gpu] c2 single pass vs forced split counts")
    o1, l1 = gpu_attention(q, k, v, w.dtype, w.scale, w.causal, splits=1)
    for s in (2, 7, 16):
        o2, l2 = gpu_attention(q, k, v, w.dtype, w.scale, w.causal, splits=s)
        # each side is within tolerance of the oracle (checked elsewhere); here they
        # must also agree with each other to the same rule
        compare(o2, l2, o1, l1, "bf16", f"c2 splits={s} vs single pass")


# ------------------------------------------------------------------ stress and special cases

def test_c4_stress_constant_v():
    # large logits with V = 1: every output is exactly 1
    w = W["c4"].with_shape(H=2, N=4096, M=4096)
    q, k, _ = si.make_qkv(w, 3)
    v = si.f32_to_bf16_bits(np.ones((w.B, w.H, w.M, w.d), dtype=np.float32))
    log("[gpu] c4-like stress, V = 1")
    o, lse = gpu_attention(q, k, v, "bf16", w.scale, True)
    # the probabilities are rounded to bf16 for the P.V product while l sums them
    # in fp32, so O may sit one bf16 step below 1
    assert np.all(np.abs(o - 1.0) <= 2.0 ** -8), f"V=1 must give O=1, max dev {np.abs(o - 1).max()}"
    rows = si.sample_rows(w, 64)
    _, lse_ref = oracle.attention_rows(si.to_f64(q, "bf16"), si.to_f64(k, "bf16"), si.to_f64(v, "bf16"),
                                       w.scale, True, rows)
    compare(o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], np.ones((len(rows), w.d)), lse_ref, "bf16",
            "c4-like V=1")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [0, 3])
def test_scores_far_below_zero(d, causal, splits):
    # Every scaled score near -300 (about -430 in base 2), a few units apart:
    # against a zero shift a row's first tile sums to 0 in fp32, so the kernel
    # must still set the row's shift from that tile (and, split over keys,
    # from the first tile of each range that holds a visible key).
    w = si.Workload("negscores", 1, 2, 300, 333, d, "bf16", causal, "normal")
    rng = np.random.default_rng(11)
    a = np.sqrt(300.0 / (d * float(w.scale)))  # q ~ a + noise, k ~ -a + noise: scale * q.k ~ -300
    q = (a + 0.3 * rng.standard_normal((w.B, w.H, w.N, d))).astype(np.float32)
    k = (-a + 0.3 * rng.standard_normal((w.B, w.H, w.M, d))).astype(np.float32)
    v = rng.standard_normal((w.B, w.H, w.M, d)).astype(np.float32)
    check_full(w, 11, splits=splits, qkv=tuple(si.f32_to_bf16_bits(x) for x in (q, k, v)))


def test_peaked_softmax_large_values():
    # Q, K with standard deviation 3 (peaked rows, the shift moves lazily, so
    # probabilities up to the tile-sum limit) and V scaled by 2^50: products
    # and sums stay finite, and O / 2^50 (an exact power-of-two scaling) meets
    # the usual rule against the oracle on the unscaled V.
    w = W["c4"].with_shape(H=2, N=1024, M=1024)
    q, k, v = si.make_qkv(w, 5)
    v_big = si.f32_to_bf16_bits(si.to_f64(v, "bf16").astype(np.float32) * np.float32(2.0 ** 50))
    log("[gpu] peaked softmax, V scaled by 2^50")
    o, lse = gpu_attention(q, k, v_big, "bf16", w.scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = oracle.attention(si.to_f64(q, "bf16"), si.to_f64(k, "bf16"), si.to_f64(v, "bf16"), w.scale, True)
    compare(o / 2.0 ** 50, lse, o_ref, lse_ref, "bf16", "peaked, V x 2^50")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_query_uniform(dtype):
    w = si.Workload("zeroq", 1, 2, 160, 300, 64, dtype, True, "normal")
    q, k, v = si.make_qkv(w, 4)
    q = np.zeros_like(q)
    check_full(w, 4, qkv=(q, k, v))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unusual_scales(scale, dtype):
    w = si.Workload("scale", 1, 2, 130, 200, 64, dtype, True, "normal")
    q, k, v = si.make_qkv(w, 9)
    log(f"[gpu] scale={scale} {dtype}")
    o, lse = gpu_attention(q, k, v, dtype, scale, True)
    o_ref, lse_ref = oracle.attention(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype),
                                      float(np.float32(scale)), True)
    bounds = None
    if dtype == "f32":
        bounds = f32_bounds(si.to_f64(q, dtype), si.to_f64(k, dtype), si.to_f64(v, dtype), float(np.float32(scale)),
                            True)
    compare(o, lse, o_ref, lse_ref, dtype, f"scale={scale}", bounds)


def test_deterministic():
    w = W["c2"].with_shape(B=1)
    q, k, v = si.make_qkv(w, 0)
    log("[gpu] run-to-run determinism")
    o1, l1 = gpu_attention(q, k, v, w.dtype, w.scale, w.causal)
    o2, l2 = gpu_attention(q, k, v, w.dtype, w.scale, w.causal)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_empty_batch_is_noop():
    import torch

    import online_softmax_10_amd as osa

    q = torch.zeros((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 3, 5, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = osa.fwd(q, k, k)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 64) and lse.shape == (2, 3, 0)


def test_binding_rejects_bad_outputs():
    # Caller-supplied outputs are checked before anything is launched.
    import torch

    import online_softmax_10_amd as osa

    log("[gpu] binding output checks")
    q = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    good_o = torch.empty_like(q)
    good_l = torch.empty((1, 2, 8), dtype=torch.float32, device="cuda")
    bad_o = [torch.empty((1, 2, 7, 64), dtype=torch.bfloat16, device="cuda"),
             torch.empty((1, 2, 8, 64), dtype=torch.float32, device="cuda"),
             torch.empty((1, 2, 64, 8), dtype=torch.bfloat16, device="cuda").transpose(2, 3),
             torch.empty((1, 2, 8, 64), dtype=torch.bfloat16)]
    for o in bad_o:
        with pytest.raises(ValueError):
            osa.fwd(q, q, q, out=o, lse=good_l)
    for l in (torch.empty((1, 2, 9), dtype=torch.float32, device="cuda"),
              torch.empty((1, 2, 8), dtype=torch.bfloat16, device="cuda")):
        with pytest.raises(ValueError):
            osa.fwd(q, q, q, out=good_o, lse=l)
    x = torch.zeros((3, 5), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        osa.online_softmax(x, out=torch.empty((3, 4), dtype=torch.float32, device="cuda"))
    o, l = osa.fwd(q, q, q, out=good_o, lse=good_l)
    torch.cuda.synchronize()
    assert o is good_o and l is good_l


# ------------------------------------------------------------------ the 256-row widths

# Shapes with at least 256 workgroups of 256 query rows, so the library runs
# a 256-row width (64 rows per wave at d = 128, eight waves at d = 64);
# ragged query and key counts (key counts off the 32- and 64-key tiles).
PINGPONG = [
    si.Workload("pp", 1, 256, 256, 300, 128, "bf16", True, "normal"),
    si.Workload("pp", 1, 256, 256, 300, 128, "bf16", False, "normal"),
    si.Workload("pp", 2, 64, 257, 513, 64, "bf16", True, "normal"),
    si.Workload("pp", 1, 128, 384, 200, 128, "bf16", True, "normal_qk3"),
    si.Workload("pp", 1, 256, 200, 1, 64, "bf16", False, "normal"),
    si.Workload("pp", 1, 256, 200, 1, 128, "bf16", False, "normal"),
    si.Workload("pp", 1, 256, 300, 33, 128, "bf16", True, "normal"),
    si.Workload("pp", 2, 128, 700, 1000, 128, "bf16", False, "normal_qk3"),
    si.Workload("pp", 1, 256, 1024, 1024, 128, "bf16", True, "normal_qk3"),
]


@pytest.mark.parametrize("w", PINGPONG, ids=[f"{w.B}x{w.H}x{w.N}x{w.M}d{w.d}{'c' if w.causal else ''}{w.dist}"
                                             for w in PINGPONG])
def test_wide_kernel_shapes(w):
    import online_softmax_10_amd as osa

    log(f"  plan {osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype)}")
    check_full(w, 21)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [0, 1])
def test_wide_kernel_scores_far_below_zero(causal, splits):
    # test_scores_far_below_zero at a size that runs the 256-row widths
    w = si.Workload("negscores", 1, 256, 300, 200, 128, "bf16", causal, "normal")
    rng = np.random.default_rng(12)
    a = np.sqrt(300.0 / (w.d * float(w.scale)))
    q = (a + 0.3 * rng.standard_normal((w.B, w.H, w.N, w.d))).astype(np.float32)
    k = (-a + 0.3 * rng.standard_normal((w.B, w.H, w.M, w.d))).astype(np.float32)
    v = rng.standard_normal((w.B, w.H, w.M, w.d)).astype(np.float32)
    check_full(w, 12, splits=splits, qkv=tuple(si.f32_to_bf16_bits(x) for x in (q, k, v)))


def test_wide_kernel_peaked_large_values():
    # test_peaked_softmax_large_values at a size that runs the 256-row widths
    w = W["c4"].with_shape(H=256, N=512, M=512)
    q, k, v = si.make_qkv(w, 6)
    v_big = si.f32_to_bf16_bits(si.to_f64(v, "bf16").astype(np.float32) * np.float32(2.0 ** 50))
    log("[gpu] peaked softmax, V scaled by 2^50, 256-row width")
    o, lse = gpu_attention(q, k, v_big, "bf16", w.scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = oracle.attention(si.to_f64(q, "bf16"), si.to_f64(k, "bf16"), si.to_f64(v, "bf16"), w.scale, True)
    compare(o / 2.0 ** 50, lse, o_ref, lse_ref, "bf16", "peaked, V x 2^50, wide")


def test_wide_kernel_constant_v():
    # V = 1 with peaked logits: O = 1 within one bf16 step, on the 256-row widths
    w = W["c4"].with_shape(H=256, N=512, M=512)
    q, k, _ = si.make_qkv(w, 7)
    v = si.f32_to_bf16_bits(np.ones((w.B, w.H, w.M, w.d), dtype=np.float32))
    log("[gpu] V = 1, 256-row width")
    o, _ = gpu_attention(q, k, v, "bf16", w.scale, True)
    assert np.all(np.abs(o - 1.0) <= 2.0 ** -8), f"V=1 must give O=1, max dev {np.abs(o - 1).max()}"


# ------------------------------------------------------------------ key halves and the four-wave single pass

# Single-pass shapes with at most 256 workgroups of 128 rows and at least 12
# (d = 64) or 16 (d = 128) 64-key tiles: each workgroup's key tiles alternate between two sets of four
# waves, merged at the end.  Odd and even tile counts, ragged tails, causal
# ranges in which the second set sees no key for the first rows, more queries
# than keys, peaked rows.
KEY_HALVES = [
    si.Workload("kh", 1, 2, 300, 1000, 64, "bf16", True, "normal"),
    si.Workload("kh", 1, 2, 300, 1000, 128, "bf16", False, "normal"),
    si.Workload("kh", 1, 4, 129, 1025, 128, "bf16", True, "normal"),
    si.Workload("kh", 1, 3, 200, 769, 64, "bf16", False, "normal_qk3"),
    si.Workload("kh", 2, 1, 900, 800, 64, "bf16", True, "normal"),
    si.Workload("kh", 2, 2, 256, 4096, 64, "bf16", True, "normal_qk3"),
    si.Workload("kh", 1, 8, 1024, 1023, 128, "bf16", True, "normal"),
]
# Single-pass shapes the four-wave kernel keeps: more than 256 workgroups of
# 128 rows but fewer than 256 of 256 rows, or fewer key tiles.
FOUR_WAVE = [
    si.Workload("w4", 1, 100, 384, 300, 64, "bf16", True, "normal"),
    si.Workload("w4", 1, 100, 300, 257, 128, "bf16", False, "normal"),
    si.Workload("w4", 1, 2, 300, 960, 128, "bf16", True, "normal"),
    si.Workload("w4", 2, 4, 500, 704, 64, "bf16", False, "normal"),
]


def _ids(ws):
    return [f"{w.B}x{w.H}x{w.N}x{w.M}d{w.d}{'c' if w.causal else ''}{w.dist}" for w in ws]


@pytest.mark.parametrize("w", KEY_HALVES, ids=_ids(KEY_HALVES))
def test_key_halves_shapes(w):
    import online_softmax_10_amd as osa

    assert osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype) == ("attn_fwd_bf16_kh_kernel", 1)
    check_full(w, 31)


@pytest.mark.parametrize("w", FOUR_WAVE, ids=_ids(FOUR_WAVE))
def test_four_wave_single_pass_shapes(w):
    import online_softmax_10_amd as osa

    assert osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype) == ("attn_fwd_bf16_kernel", 1)
    check_full(w, 32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_key_halves_scores_far_below_zero(d, causal):
    # test_scores_far_below_zero on the key-halves kernel: each set of waves
    # sets its rows' shifts from its own first tile
    import online_softmax_10_amd as osa

    w = si.Workload("negscores", 1, 2, 300, 1100, d, "bf16", causal, "normal")
    assert osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype)[0] == "attn_fwd_bf16_kh_kernel"
    rng = np.random.default_rng(13)
    a = np.sqrt(300.0 / (d * float(w.scale)))
    q = (a + 0.3 * rng.standard_normal((w.B, w.H, w.N, d))).astype(np.float32)
    k = (-a + 0.3 * rng.standard_normal((w.B, w.H, w.M, d))).astype(np.float32)
    v = rng.standard_normal((w.B, w.H, w.M, d)).astype(np.float32)
    check_full(w, 13, qkv=tuple(si.f32_to_bf16_bits(x) for x in (q, k, v)))


def test_key_halves_peaked_large_values():
    # test_peaked_softmax_large_values on the key-halves kernel: the two sets
    # of waves reach different shifts, which the merge reconciles
    import online_softmax_10_amd as osa

    w = W["c4"].with_shape(H=4, N=512, M=2048)
    assert osa.plan(w.B, w.H, w.N, w.M, w.d, w.dtype)[0] == "attn_fwd_bf16_kh_kernel"
    q, k, v = si.make_qkv(w, 8)
    v_big = si.f32_to_bf16_bits(si.to_f64(v, "bf16").astype(np.float32) * np.float32(2.0 ** 50))
    log("[gpu] peaked softmax, V scaled by 2^50, key halves")
    o, lse = gpu_attention(q, k, v_big, "bf16", w.scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = oracle.attention(si.to_f64(q, "bf16"), si.to_f64(k, "bf16"), si.to_f64(v, "bf16"), w.scale, True)
    compare(o / 2.0 ** 50, lse, o_ref, lse_ref, "bf16", "peaked, V x 2^50, key halves")
