"""Comparison helpers for GPU-vs-oracle parity (no attention arithmetic here).

Tolerances (the bar for every parity test):
  * outputs in fp16: |gpu - oracle| <= 2e-3
  * outputs in bf16: |gpu - oracle| <= 1e-2
  * LSE (float32):  |gpu - oracle| <= 1e-3
  * float32 partial outputs (before the final rounding): <= 1e-3
Rounding the exact result to fp16/bf16 alone moves it by up to half the
type's spacing at that value, which exceeds the absolute bound wherever
|O| >= 8 (fp16) or >= 4 (bf16): only such elements (half a spacing above the
bound, seen with the 8x outlier rows) get one spacing on top of the bound.
strict=True drops that allowance everywhere (plain max-abs), for workloads
whose outputs stay below those magnitudes.
Rows with no keys must be exactly O = 0, LSE = -inf.
"""
import os

import numpy as np
import torch

from split_kv_paged_amd import workloads as W

ATOL = {"fp16": 2e-3, "bf16": 1e-2}
LSE_ATOL = 1e-3
PART_ATOL = 1e-3
TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}

# (test id, what, max abs error, bar) of every passing check, for the raw
# error table that tests/conftest.py prints after a run
RECORDS = []


def _record(what, err, bar):
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    RECORDS.append((test, what, err, bar))


def to_dev(bits, dtype, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def i32_dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def bits_of(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def ulp(x, dtype):
    a = np.abs(np.asarray(x, dtype=np.float64))
    if dtype == "fp16":
        a16 = np.minimum(a, 65504.0).astype(np.float16)
        return np.spacing(a16).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def allowance(ref, dtype, strict=False):
    """Per-element bound: the absolute bar, plus one spacing of the output
    type where half a spacing exceeds the bar (never with strict)."""
    ref = np.asarray(ref, dtype=np.float64)
    allow = np.full(ref.shape, ATOL[dtype])
    if not strict:
        sp = ulp(ref, dtype)
        allow = np.where(0.5 * sp > ATOL[dtype], ATOL[dtype] + sp, allow)
    return allow


def check_out(got_bits, ref, dtype, what="out", strict=False):
    got = W.from_bits(got_bits, dtype).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = np.abs(got - ref)
    allow = allowance(ref, dtype, strict)
    bad = err > allow
    if bad.any():
        idx = np.unravel_index(np.argmax(err - allow), err.shape)
        raise AssertionError("%s: %d/%d elements out of tolerance; worst at %s: gpu %r oracle %r "
                             "(max abs err %.3g)" % (what, bad.sum(), err.size, idx, got[idx],
                                                     ref[idx], err.max()))
    worst = float(err.max()) if err.size else 0.0
    _record(what, worst, ATOL[dtype] if strict else "%g+spacing" % ATOL[dtype])
    return worst


def check_lse(got, ref, what="lse", atol=LSE_ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), "%s: -inf pattern differs" % what
    if (~empty).any():
        err = np.abs(got[~empty] - ref[~empty])
        assert err.max() <= atol, "%s: max err %.3g" % (what, err.max())
        _record(what, float(err.max()), atol)
        return float(err.max())
    return 0.0


def check_f32(got, ref, atol=PART_ATOL, what="partial"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), what
    assert err.max(initial=0.0) <= atol, "%s: max err %.3g" % (what, err.max())
    return float(err.max(initial=0.0))
