"""GPU parity of the row-wise online_softmax (through the C ABI) against the
float64 three-pass oracle, and the pages' worked example."""

import json
import math
import os

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity import F32_TOL, log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gpu_softmax(x: np.ndarray) -> np.ndarray:
    import torch

    import online_softmax_10_amd as osa

    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    y = osa.online_softmax(xd)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def test_c1_softmax_row_worked_example():
    with open(os.path.join(GOLDEN, "w1_softmax.json"), encoding="utf-8") as f:
        g = json.load(f)
    log("[gpu] online_softmax on the worked-example logits")
    x = si.C1_SOFTMAX_ROW
    y = gpu_softmax(x)
    ref = oracle.softmax(x.astype(np.float64))
    assert np.max(np.abs(y - ref)) <= F32_TOL, (y, ref)
    assert np.max(np.abs(y[0] - np.array(g["softmax"]))) <= g["tol_printed"]
    # cross-entropy for class 0 from the device probabilities (the second worked example)
    with open(os.path.join(GOLDEN, "w2_cross_entropy.json"), encoding="utf-8") as f:
        g2 = json.load(f)
    assert abs(-math.log(y[0, 0]) - g2["loss"]) <= g2["tol_printed"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 63, 64, 65, 256, 260, 512, 1000, 2048, 3000, 4096, 4097, 4100,
                               8192, 12000, 16388, 32768, 50000, 65536, 65540, 70000])
def test_rows_match_oracle(n):
    rows = 37 if n <= 4096 else 5
    x = si.make_rows(rows, n, seed=n, spread=4.0)
    log(f"[gpu] online_softmax rows={rows} n={n}")
    y = gpu_softmax(x)
    ref = oracle.softmax(x.astype(np.float64))
    err = np.max(np.abs(y - ref))
    log(f"  max|dy|={err:.3e}")
    assert err <= F32_TOL
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) <= 1e-5


def test_large_logits_and_neg_inf():
    x = si.make_rows(6, 300, seed=3, spread=1.0)
    x[0] += 1000.0          # would overflow e^x without the max shift
    x[1] -= 1000.0
    x[2, ::3] = -np.inf     # masked entries give exactly 0
    x[3, 0] = 80.0          # one dominant logit
    log("[gpu] online_softmax large logits / -inf entries")
    y = gpu_softmax(x)
    ref = oracle.softmax(x.astype(np.float64))
    assert np.all(np.isfinite(y))
    assert np.max(np.abs(y - ref)) <= F32_TOL
    assert np.all(y[2, ::3] == 0.0)


@pytest.mark.parametrize("n", [300, 6000, 70000])
def test_huge_logits(n):
    # Logits far beyond any exponent range: only differences matter.
    x = si.make_rows(5, n, seed=4, spread=1.0)
    x[0, :] = -1e30                 # all equal and huge: uniform
    x[1, :] = 3e37
    x[2, :] = np.float32(1e30) * np.sign(x[2, :])  # two distinct values 2e30 apart: one-hot on the positive ones
    x[3] *= np.float32(1e6)         # spread of a million
    x[4, 7] = 1e38
    log(f"[gpu] online_softmax huge logits n={n}")
    y = gpu_softmax(x)
    ref = oracle.softmax(x.astype(np.float64))
    assert np.all(np.isfinite(y))
    assert np.max(np.abs(y - ref)) <= F32_TOL


def test_many_rows_and_in_place():
    import torch

    import online_softmax_10_amd as osa

    x = si.make_rows(300000, 12, seed=5, spread=2.0)
    log("[gpu] online_softmax 300000 x 12, in place")
    xd = torch.from_numpy(x).cuda()
    osa.online_softmax(xd, out=xd)
    torch.cuda.synchronize()
    y = xd.cpu().numpy().astype(np.float64)
    ref = oracle.softmax(x.astype(np.float64))
    assert np.max(np.abs(y - ref)) <= F32_TOL


@pytest.mark.parametrize("n", [1, 3, 64, 260, 1000, 4096, 4097, 8192, 32768, 65536, 70000])
def test_lse_matches_oracle(n):
    # online_softmax_lse: softmax rows and their log-sum-exp together, and the
    # log-sum-exp alone (one read of x), on every kernel path.
    import torch

    import online_softmax_10_amd as osa

    rows = 37 if n <= 4096 else 5
    x = si.make_rows(rows, n, seed=100 + n, spread=4.0)
    x[0] += 500.0  # far above any exponent range: only differences enter
    log(f"[gpu] online_softmax_lse rows={rows} n={n}")
    xd = torch.from_numpy(x).cuda()
    y, lse = osa.online_softmax(xd, return_lse=True)
    lse_only = osa.logsumexp(xd)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    lse_only = lse_only.cpu().numpy().astype(np.float64)
    ref_y = oracle.softmax(x.astype(np.float64))
    ref_lse = oracle.logsumexp(x.astype(np.float64))
    # The LSE is an fp32 number of the logits' size formed by a few fp32
    # additions (m + log s): each rounds by at most u times that size, so the
    # bound is 1e-5 + 3u max|x| (u = 2^-24).
    tol = F32_TOL + 3 * 2.0 ** -24 * np.abs(x).max(axis=1)
    dl = np.abs(lse - ref_lse)
    log(f"  max|dlse|={dl.max():.3e} (row bound {tol.min():.1e}..{tol.max():.1e}) max|dy|={np.abs(y - ref_y).max():.3e}")
    assert np.all(dl <= tol)
    assert np.array_equal(lse, lse_only), "the LSE alone must equal the LSE given with the softmax"
    assert np.max(np.abs(y - ref_y)) <= F32_TOL


def test_lse_of_neg_inf_row():
    import torch

    import online_softmax_10_amd as osa

    x = si.make_rows(3, 100, seed=9)
    x[1, :] = -np.inf
    x[2, 5:] = -np.inf
    log("[gpu] logsumexp with an all -inf row")
    lse = osa.logsumexp(torch.from_numpy(x).cuda()).cpu().numpy().astype(np.float64)
    assert np.isneginf(lse[1])
    ref = oracle.logsumexp(x[[0, 2]].astype(np.float64))
    assert np.max(np.abs(lse[[0, 2]] - ref)) <= F32_TOL
