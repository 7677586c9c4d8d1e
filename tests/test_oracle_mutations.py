"""Plant plausible mistakes in a copy of the oracle and check the pins fail.

Each mutation edits the C source text of a temporary copy (the committed
oracle is never touched), builds it with gcc, routes the oracle through it
and runs the pin tests.  A mutation that no pin catches fails this test.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# (name, original text, planted mistake)
MUTATIONS = [
    ("scale dropped", "s[j - j0] = P->scale * acc;", "s[j - j0] = acc;"),
    ("lse in log2", "*lse = m + log(l);\n    free(s);", "*lse = m + log2(l);\n    free(s);"),
    ("no max offset in the sum", "for (j = j0; j < j1; ++j) l += exp(s[j - j0] - m);",
     "for (j = j0; j < j1; ++j) l += exp(s[j - j0]);"),
    ("kv head by modulo", "h = hh / G;", "h = hh % hkv;"),
    ("paged head by modulo", "int hh = h * G + g;", "int hh = g * hkv + h;"),
    ("page slot swapped", "long off = ((page * page_size + j % page_size) * hkv + h) * (long)d;",
     "long off = ((page * page_size + j / page_size % page_size) * hkv + h) * (long)d;"),
    ("online: no rescale", "for (e = 0; e < d; ++e) o[e] *= alpha;", ""),
    ("online: old sum kept", "l = alpha * l + exp(bmax - m_new) * bsum;",
     "l = l + exp(bmax - m_new) * bsum;"),
    ("combine: unnormalised", "for (e = 0; e < d; ++e) o[e] /= wsum;", ""),
    ("combine: lse without shift", "lse[n] = M + log(wsum);", "lse[n] = log(wsum);"),
    ("split ranges overlap", "long a = (long)s * C, b = (long)(s + 1) * C;",
     "long a = (long)s * C, b = (long)(s + 2) * C;"),
    ("split ranges leave gaps", "long a = (long)s * C, b = (long)(s + 1) * C;",
     "long a = (long)s * C + 1, b = (long)(s + 1) * C;"),
    ("fp16 subnormal scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("bf16 exponent bias", "v = ldexp((double)(128 + f), e - 134);",
     "v = ldexp((double)(128 + f), e - 133);"),
    ("causal off by one", "n = L - qlen + 1 + i;", "n = L - qlen + i;"),
    ("causal top-left aligned", "n = L - qlen + 1 + i;", "n = 1 + i;"),
    ("empty sequence lse", "if (j1 <= j0) {\n        *lse = -INFINITY;\n        return;\n    }\n    s =",
     "if (j1 <= j0) {\n        *lse = 0.0;\n        return;\n    }\n    s ="),
]

PIN_TESTS = [
    (pins.test_decode_fp16_all_patterns, {}),
    (pins.test_decode_bf16_all_patterns, {}),
    (pins.test_single_key_gives_value_row, {}),
    (pins.test_identical_keys_give_mean_value, {}),
    (pins.test_two_keys_logistic_weights, {}),
    (pins.test_dominant_key_selects_its_value, {}),
    (pins.test_empty_sequence_gives_zero_and_minus_inf, {}),
    (pins.test_dense_matches_torch_sdpa, dict(dtype="bf16", hq=8, hkv=2, qlen=2, L=33, d=64)),
    (pins.test_paged_matches_torch_sdpa_on_gathered_kv, dict(dtype="bf16", G=4, d=128, page=16)),
    (pins.test_paged_matches_torch_sdpa_on_gathered_kv, dict(dtype="fp16", G=1, d=32, page=5)),
    (pins.test_value_and_lse_bounds, {}),
    (pins.test_split_partials_and_combine_equal_direct, dict(block=5)),
    (pins.test_split_ranges_cover_keys_once_and_empty_splits_are_neutral, {}),
    (pins.test_combine_closed_forms, {}),
    (pins.test_causal_dense_matches_torch_with_bottom_right_mask,
     dict(hq=8, hkv=2, qlen=4, L=33, d=64)),
    (pins.test_causal_closed_forms, {}),
]


def _build_variant(text, tmpdir, tag):
    src = os.path.join(tmpdir, "mut_%s.c" % tag)
    lib = os.path.join(tmpdir, "libmut_%s.so" % tag)
    with open(src, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-D_DEFAULT_SOURCE", "-w", "-shared", "-fPIC",
                           "-pthread", src, "-o", lib, "-lm"])
    return lib


def _caught(lib):
    with oracle.use_library(lib):
        for fn, kw in PIN_TESTS:
            try:
                fn(**kw)
            except (AssertionError, ValueError, FloatingPointError):
                return fn.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation anchor not found once: %r" % old
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_variant(text.replace(old, new), tmp, "x")
        assert _caught(lib) is not None, "no pin caught the planted mistake: %s" % name


def test_unmutated_copy_passes_every_pin():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_variant(text, tmp, "clean")
        assert _caught(lib) is None
