"""The pins are sensitive: each plausible mistake planted in a copy of the
oracle's C source (on the CPU, in a temporary directory) fails at least one pin.
"""

import os
import shutil

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted text); each original occurs exactly once.
MUTATIONS = [
    ("dropped scale", "s[j] = scale * acc;", "s[j] = acc;"),
    ("dropped first term of the sum",
     "for (int64_t j = 0; j < visible; ++j)\n                l += exp(s[j] - m);",
     "for (int64_t j = 1; j < visible; ++j)\n                l += exp(s[j] - m);"),
    ("wrong sign in the weight", "double p = exp(s[j] - m) / l;", "double p = exp(m - s[j]) / l;"),
    ("causal off by one", "if (causal_mode == 1 && i + 1 < visible) visible = i + 1;",
     "if (causal_mode == 1 && i + 2 < visible) visible = i + 2;"),
    ("bottom-right mask without the offset",
     "if (causal_mode == 2 && i + 1 + (M - N) < visible) visible = i + 1 + (M - N) > 0 ? i + 1 + (M - N) : 0;",
     "if (causal_mode == 2 && i + 1 < visible) visible = i + 1;"),
    ("key lengths ignored", "if (kv_len && kv_len[bh / H] < visible)", "if (0 && kv_len && kv_len[bh / H] < visible)"),
    ("key length of the wrong batch", "visible = kv_len[bh / H] > 0 ? kv_len[bh / H] : 0;",
     "visible = kv_len[0] > 0 ? kv_len[0] : 0;"),
    ("empty row LSE of 0", "lse_rows[t] = -INFINITY;", "lse_rows[t] = 0.0;"),
    ("bias subtracted", "s[j] += brow[j];", "s[j] -= brow[j];"),
    ("bias scaled with the product", "s[j] += brow[j];", "s[j] += scale * brow[j];"),
    ("bias of head 0 for every head", "(bh % H) * bias_sh", "0 * bias_sh"),
    ("bias rows of query 0", "i * bias_sn : NULL;", "0 * bias_sn : NULL;"),
    ("all -inf row not caught", "if (m == -INFINITY) {", "if (0) {"),
    ("K used in place of V", "oi[c] += p * vh[j * d + c];", "oi[c] += p * kh[j * d + c];"),
    ("reversed feature index", "acc += qi[c] * kh[j * d + c];", "acc += qi[c] * kh[j * d + (d - 1 - c)];"),
    ("LSE without the max", "lse_rows[t] = m + log(l);", "lse_rows[t] = log(l);"),
    ("softmax without the divide", "yr[j] = exp(xr[j] - m) / s;", "yr[j] = exp(xr[j] - m);"),
    ("softmax shifts by the min",
     "double *yr = y + r * n;\n        /* pass 1: the maximum */\n        double m = xr[0];\n"
     "        for (int64_t j = 1; j < n; ++j)\n            if (xr[j] > m) m = xr[j];",
     "double *yr = y + r * n;\n        /* pass 1: the maximum */\n        double m = xr[0];\n"
     "        for (int64_t j = 1; j < n; ++j)\n            if (xr[j] < m) m = xr[j];"),
    ("normaliser without the rescale", "const double carried = m == -INFINITY ? 0.0 : s * exp(m - m_next);",
     "const double carried = m == -INFINITY ? 0.0 : s;"),
    ("normaliser rescale inverted", "const double carried = m == -INFINITY ? 0.0 : s * exp(m - m_next);",
     "const double carried = m == -INFINITY ? 0.0 : s * exp(m_next - m);"),
    ("normaliser's empty prefix with maximum 0", "double m = -INFINITY; /* the empty prefix */",
     "double m = 0.0; /* the empty prefix */"),
    ("LSE of softmax rows without the max", "lse[r] = m + log(s);", "lse[r] = log(s);"),
    ("query row ignores the head", "const double *qi = q + r * d;", "const double *qi = q + i * d;"),
    ("every head uses head 0's keys", "const double *kh = k + bh * M * d;", "const double *kh = k;"),
    ("cross-entropy sign flipped", "loss[r] = -log_prob;", "loss[r] = log_prob;"),
    ("cross-entropy label off by one", "const double log_prob = xr[c] - m - log_sum;",
     "const double log_prob = xr[(c + 1) % n] - m - log_sum;"),
    ("cross-entropy without the max", "const double log_prob = xr[c] - m - log_sum;",
     "const double log_prob = xr[c] - log_sum;"),
    ("cross-entropy LSE without the max", "lse[r] = m + log_sum;", "lse[r] = log_sum;"),
    ("cross-entropy invalid label scored", "loss[r] = NAN;", "loss[r] = 0.0;"),
]


@pytest.mark.parametrize("name,orig,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, orig, planted, tmp_path):
    with open(SRC, encoding="utf-8") as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation anchor for {name!r} must occur exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(orig, planted), encoding="utf-8")
    so = oracle.build(out=str(tmp_path / "liboracle_mutant.so"), src=str(mutant), extra_flags=("-w",))
    lib = oracle.load(so)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            failures.append((pin.__name__, str(e).splitlines()[0]))
    assert failures, f"planted mistake {name!r} passed every pin"
    shutil.rmtree(tmp_path, ignore_errors=True)
