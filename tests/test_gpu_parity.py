"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every test prints the case it is about to run (flushed) before its first
GPU call.  Full-size cases use the five named workloads; small cases span
several 16-key tiles with ragged tails, GQA 1/2/4/8, q_len up to 8 (row
blocks), head_dim 1..256, both dtypes, page sizes 16/32/48, empty sequences
and NaN-poisoned slots outside the valid keys.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from split_kv_paged_amd import api
from split_kv_paged_amd import workloads as W
from tests.parity import (bits_of, check_f32, check_lse, check_out, i32_dev, to_dev)

pytestmark = pytest.mark.gpu


def case(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


def run_paged(wl, num_splits=0, pack_gqa=-1, workspace=None, sum_hint=False):
    q = to_dev(wl.q, wl.dtype)
    kc = to_dev(wl.k_cache, wl.dtype)
    vc = to_dev(wl.v_cache, wl.dtype)
    bt = i32_dev(wl.block_table)
    sl = i32_dev(wl.cache_seqlens)
    out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=num_splits, pack_gqa=pack_gqa,
                              softmax_scale=wl.scale, max_seqlen_k=max(wl.max_seqlen_k, 0),
                              workspace=workspace,
                              sum_seqlen_k=int(wl.cache_seqlens.sum()) if sum_hint else None)
    torch.cuda.synchronize()
    return bits_of(out), lse.cpu().numpy(), api.last_plan()


def oracle_paged(wl):
    return oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                  wl.cache_seqlens, wl.dtype, scale=wl.scale)


def assert_paged(wl, num_splits=0, pack_gqa=-1, ref=None, strict=False, sum_hint=False):
    """strict: the plain max-abs bar (for N(0,1) workloads, whose outputs
    stay far below the magnitudes where rounding alone would exceed it)."""
    ref_o, ref_l = ref if ref is not None else oracle_paged(wl)
    out, lse, plan = run_paged(wl, num_splits, pack_gqa, sum_hint=sum_hint)
    e1 = check_out(out, ref_o, wl.dtype, "%s S=%d" % (wl.name, num_splits), strict=strict)
    e2 = check_lse(lse, ref_l)
    print("  plan S=%d pack=%d rows/blk=%d grid=%d heads/row=%d extra=%d  raw max|dO|=%.3g "
          "max|dLSE|=%.3g (bar %s)" % (
              plan.num_splits, plan.pack_gqa, plan.rows_per_block, plan.grid, plan.heads_per_row,
              plan.extra_blocks, e1, e2, "plain" if strict else "plain + spacing above 0.5 ulp"),
          flush=True)
    return plan


# ---------------------------------------------------------------- workloads --

@pytest.fixture(scope="module")
def c3():
    wl = W.c3_paged_gqa4()
    return wl, oracle_paged(wl)


def test_paged_gqa4_bf16_full_size_planner(c3):
    wl, ref = c3
    case("paged bf16 B32 Hq32/Hkv8 d128 L~U[900,1100], planner splits")
    plan = assert_paged(wl, ref=ref, strict=True)
    assert plan.num_splits == 1 and plan.pack_gqa == 1


def test_paged_gqa4_bf16_bench_path(c3):
    """The call the benchmark times: the planner with the length sum given."""
    wl, ref = c3
    case("paged bf16 B32 Hq32/Hkv8 d128 L~U[900,1100], planner with the length sum")
    plan = assert_paged(wl, ref=ref, strict=True, sum_hint=True)
    assert plan.num_splits == 1 and plan.pack_gqa == 1 and plan.extra_blocks == 0


@pytest.mark.parametrize("S", [2, 3, 4, 8])
def test_paged_gqa4_bf16_full_size_split_sweep(c3, S):
    wl, ref = c3
    case("paged bf16 B32 Hq32/Hkv8 d128, num_splits=%d" % S)
    plan = assert_paged(wl, num_splits=S, ref=ref, strict=True)
    assert plan.num_splits == S and plan.combine >= 1


def test_paged_gqa4_bf16_full_size_unpacked(c3):
    wl, ref = c3
    case("paged bf16 B32 Hq32/Hkv8 d128, pack_gqa=0")
    plan = assert_paged(wl, num_splits=1, pack_gqa=0, ref=ref, strict=True)
    assert plan.pack_gqa == 0 and plan.rows_per_unit == 1


@pytest.fixture(scope="module")
def c4():
    wl = W.c4_long()
    return wl, oracle_paged(wl)


@pytest.mark.parametrize("S", [0, 1, 2, 4, 8, 16])
def test_long_context_bf16_split_sweep(c4, S):
    wl, ref = c4
    case("paged bf16 B4 Hq32/Hkv4 d128 L16384, num_splits=%d" % S)
    plan = assert_paged(wl, num_splits=S, ref=ref, strict=True)
    if S == 0:
        assert plan.num_splits == 14


def test_long_context_bf16_bench_path(c4):
    """The call the benchmark times: the planner with the length sum given
    (a uniform batch: the pages' rule's S = 14 raised to fill the 256 CUs,
    S = 16, fused combine)."""
    wl, ref = c4
    case("paged bf16 B4 Hq32/Hkv4 d128 L16384, planner with the length sum")
    plan = assert_paged(wl, ref=ref, strict=True, sum_hint=True)
    assert plan.num_splits == 16 and plan.combine == 2


def test_ragged_fp16_outliers_full_size():
    wl = W.c5_ragged()
    case("paged fp16 B128 Hq16/Hkv8 d64 L log-uniform 1..8192, 1%% outliers x8 (%d rows)"
         % wl.meta["outlier_rows"])
    ref = oracle_paged(wl)
    assert_paged(wl, ref=ref)
    case("same, num_splits=8")
    assert_paged(wl, num_splits=8, ref=ref)


def test_ragged_fp16_outliers_bench_path():
    """The call the benchmark times on the ragged workload: its 1% x8 outlier
    rows, the planner with the length sum (ragged splits, head pairs, the
    compact split list)."""
    wl = W.c5_ragged()
    case("paged fp16 B128 Hq16/Hkv8 d64 L log-uniform 1..8192, 1%% outliers x8 (%d rows), "
         "planner with the length sum" % wl.meta["outlier_rows"])
    plan = assert_paged(wl, sum_hint=True)
    assert plan.num_splits == 8 and plan.heads_per_row == 2 and plan.extra_blocks > 0


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("S", [1, 4])
def test_paged_outliers_full_size(dt, S):
    """The paged GQA-4 d 128 shape with 1% of K/V rows scaled by 8: large,
    cancelling P.V terms, where 16-bit probabilities rounded once fall
    outside the tolerance in both types (the kernel adds their residue)."""
    rng = np.random.default_rng(1003)
    lens = [int(x) for x in rng.integers(900, 1101, 32)]
    wl = W.make_paged(1903, dt, 32, 1, 32, 8, 128, 16, lens, spare_pages=1, outlier_p=0.01)
    case("paged %s B32 GQA-4 d128 L~1000, 1%% outliers x8 (%d rows), S=%d"
         % (dt, wl.meta["outlier_rows"], S))
    assert_paged(wl, num_splits=S)


# One batch holding sequence lengths from 1 to 8192 (tile edges and their
# neighbours), over the pages' supported grid (fp16 and bf16, head dim 64 and
# 128, GQA 2/4/8).  "ovf" widens the logits 30-fold through the softmax
# scale: scores then reach about +-120, whose exponentials overflow float32
# unless the running maximum is taken off first.
MATRIX_LENS = [1, 2, 15, 16, 17, 255, 1023, 1025, 4096, 8191, 8192]


@pytest.mark.parametrize("ovf", [False, True], ids=["n01", "ovf"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_robustness_matrix(dt, G, d, ovf):
    """The MXFlashAttn page's robustness matrix (section 快速复现: lengths 1
    to 8192, GQA 2/4/8, bf16, overflow) over the shapes of its 能力矩阵
    table, each case called three ways: the pages' split rule, the rule with
    the length sum (ragged splits; head pairs at d 64) and four splits."""
    scale = (30.0 if ovf else 1.0) / np.sqrt(d)
    seed = 7100 + 8 * d + G + (1000 if ovf else 0) + (500 if dt == "fp16" else 0)
    wl = W.make_paged(seed, dt, len(MATRIX_LENS), 1, 2 * G, 2, d, 16, MATRIX_LENS,
                      spare_pages=2, scale=scale,
                      name="matrix-%s-G%d-d%d-%s" % (dt, G, d, "ovf" if ovf else "n01"))
    case("%s: lengths %s, softmax scale %.4g" % (wl.name, MATRIX_LENS, scale))
    ref = oracle_paged(wl)
    if ovf:  # the premise: some row's log-sum-exp lies beyond float32's exp range
        assert ref[1].max() > 89.0, ref[1].max()
    for S, hint in ((0, False), (0, True), (4, False)):
        assert_paged(wl, num_splits=S, ref=ref, sum_hint=hint)


def test_dense_decode_fp16():
    wl = W.c1_dense_decode()
    case("dense fp16 Hq8/Hkv2 d64 kvLen512 scale 1/8, num_splits=1")
    ref_o, ref_l = oracle.dense_attention(wl.q, wl.k, wl.v, "fp16", scale=wl.scale)
    out, lse = api.dense_fwd(to_dev(wl.q, "fp16"), to_dev(wl.k, "fp16"), to_dev(wl.v, "fp16"),
                             num_splits=1, softmax_scale=wl.scale)
    torch.cuda.synchronize()
    e1 = check_out(bits_of(out), ref_o, "fp16", strict=True)
    check_lse(lse.cpu().numpy(), ref_l)
    assert api.last_plan().num_splits == 1
    print("  raw max|dO|=%.3g (plain bar 2e-3)" % e1, flush=True)


@pytest.mark.parametrize("kv_len", W.C2_KV_LENS)
def test_smallq_mha_fp16(kv_len):
    wl = W.c2_smallq(kv_len)
    case("dense fp16 MHA 32 heads qLen4 d128 kvLen=%d, planner splits" % kv_len)
    ref_o, ref_l = oracle.dense_attention(wl.q, wl.k, wl.v, "fp16")
    q, k, v = to_dev(wl.q, "fp16"), to_dev(wl.k, "fp16"), to_dev(wl.v, "fp16")
    out, lse = api.dense_fwd(q, k, v)
    torch.cuda.synchronize()
    plan = api.last_plan()
    e1 = check_out(bits_of(out), ref_o, "fp16", strict=True)
    check_lse(lse.cpu().numpy(), ref_l)
    print("  planner S=%d raw max|dO|=%.3g (plain bar 2e-3)" % (plan.num_splits, e1), flush=True)
    if kv_len == 1:  # one key: O is that value row, exactly
        np.testing.assert_array_equal(bits_of(out), np.broadcast_to(wl.v, out.shape))
    for S in (1, 3):
        case("dense fp16 MHA kvLen=%d num_splits=%d" % (kv_len, S))
        out, lse = api.dense_fwd(q, k, v, num_splits=S)
        torch.cuda.synchronize()
        check_out(bits_of(out), ref_o, "fp16", strict=True)
        check_lse(lse.cpu().numpy(), ref_l)


@pytest.mark.parametrize("ovf", [False, True], ids=["n01", "ovf"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_dense_robustness_matrix(dt, d, G, ovf):
    """The robustness matrix on the dense small-query path (q_len 4): kvLen
    1, 17, 1025 and 8192, MHA and GQA 2/4/8, both types, with N(0,1) logits
    and with logits widened 30-fold ("ovf", as for the paged matrix); the
    planner's split count and three splits."""
    scale = (30.0 if ovf else 1.0) / np.sqrt(d)
    for kv_len in (1, 17, 1025, 8192):
        seed = 7300 + kv_len + 4 * d + G + (100 if ovf else 0) + (50 if dt == "fp16" else 0)
        wl = W.make_dense(seed, dt, 2 * G, 2, 4, kv_len, d, scale=scale)
        ref_o, ref_l = oracle.dense_attention(wl.q, wl.k, wl.v, dt, scale=scale)
        if ovf and kv_len >= 1025:  # the premise, as for the paged matrix
            assert ref_l.max() > 89.0, ref_l.max()
        q, k, v = to_dev(wl.q, dt), to_dev(wl.k, dt), to_dev(wl.v, dt)
        for S in (0, 3):
            case("dense %s Hq%d/Hkv2 q4 kvLen %d d%d scale %.4g S=%d" % (dt, 2 * G, kv_len, d,
                                                                         scale, S))
            out, lse = api.dense_fwd(q, k, v, num_splits=S, softmax_scale=scale)
            torch.cuda.synchronize()
            check_out(bits_of(out), ref_o, dt)
            check_lse(lse.cpu().numpy(), ref_l)


DENSE_ROWS = [
    # dtype, Hq, Hkv, q_len, kv_len, d: packed rows G * q_len per unit
    ("bf16", 8, 8, 40, 700, 128),    # MHA, 40 rows: a 64-row block (Q staged in LDS)
    ("fp16", 16, 2, 8, 1500, 128),   # GQA 8, 64 rows
    ("bf16", 4, 1, 24, 300, 64),     # MQA, 96 rows: two 64-row blocks at d 64
    ("fp16", 8, 4, 12, 999, 128),    # GQA 2, 24 rows: one 32-row block
]


@pytest.mark.parametrize("spec", DENSE_ROWS, ids=lambda s: "%s-G%d-q%d-d%d" % (
    s[0], s[1] // s[2], s[3], s[5]))
@pytest.mark.parametrize("S", [0, 1, 4])
def test_dense_many_rows(spec, S):
    """The dense small-query path with units of more than 16 rows (32- and
    64-row workgroups)."""
    dt, hq, hkv, qlen, kvlen, d = spec
    wl = W.make_dense(2100 + qlen + d, dt, hq, hkv, qlen, kvlen, d)
    case("dense %s Hq%d/Hkv%d q%d kvLen %d d%d S=%d" % (dt, hq, hkv, qlen, kvlen, d, S))
    ref_o, ref_l = oracle.dense_attention(wl.q, wl.k, wl.v, dt, scale=wl.scale)
    out, lse = api.dense_fwd(to_dev(wl.q, dt), to_dev(wl.k, dt), to_dev(wl.v, dt), num_splits=S,
                             softmax_scale=wl.scale)
    torch.cuda.synchronize()
    check_out(bits_of(out), ref_o, dt)
    check_lse(lse.cpu().numpy(), ref_l)
    print("  plan S=%d rows/blk=%d grid=%d" % (api.last_plan().num_splits,
                                               api.last_plan().rows_per_block,
                                               api.last_plan().grid), flush=True)


# ---------------------------------------------------------- any head_dim ----

ODD_DIMS = [1, 7, 16, 24, 33, 48, 80, 96, 100, 112, 130, 160, 192, 200, 255, 256, 32]


@pytest.mark.parametrize("d", ODD_DIMS)
def test_dense_any_head_dim(d):
    """Row a11's arbitrary head dim: padded tiles, element loads, masked
    stores (head dims 32/64/128/256 take the 16-byte path)."""
    dt = "bf16" if d % 2 else "fp16"
    wl = W.make_dense(900 + d, dt, 8, 2, 3, 301, d)
    ref_o, ref_l = oracle.dense_attention(wl.q, wl.k, wl.v, dt, scale=wl.scale)
    q, k, v = to_dev(wl.q, dt), to_dev(wl.k, dt), to_dev(wl.v, dt)
    for S in (1, 4):
        case("dense %s Hq8/Hkv2 qLen3 kvLen301 head_dim=%d num_splits=%d" % (dt, d, S))
        out, lse = api.dense_fwd(q, k, v, num_splits=S)
        torch.cuda.synchronize()
        check_out(bits_of(out), ref_o, dt)
        check_lse(lse.cpu().numpy(), ref_l)
        assert api.last_plan().kernel % 1000 >= d


@pytest.mark.parametrize("d", [32, 80, 96, 256])
def test_paged_any_head_dim(d):
    wl = W.make_paged(950 + d, "bf16", 3, 2, 8, 2, d, 16, [5, 130, 47], spare_pages=2)
    ref = oracle_paged(wl)
    for S in (1, 3):
        case("paged bf16 B3 q2 Hq8/Hkv2 head_dim=%d S=%d" % (d, S))
        assert_paged(wl, num_splits=S, ref=ref)


# ------------------------------------------- causal small-q and KV append ----

CAUSAL = [
    # dtype, B, qlen, Hq, Hkv, d, lens
    ("bf16", 3, 4, 32, 8, 128, [2, 4, 300]),     # GQA 4: 16 rows; L < q_len; L = q_len
    ("fp16", 2, 8, 16, 2, 64, [9, 129]),         # GQA 8 d 64: one 64-row block
    ("bf16", 2, 2, 8, 8, 128, [1, 77]),          # MHA, one query sees nothing in b 0
    ("fp16", 2, 3, 8, 4, 96, [40, 1000]),        # any head dim
    ("bf16", 2, 5, 8, 1, 64, [17, 18]),          # MQA, 40 rows
    ("bf16", 2, 8, 64, 8, 128, [33, 700]),       # GQA 8 d 128: one 64-row block (Q in LDS)
    ("fp16", 2, 6, 64, 8, 128, [1, 500]),        # 48 rows: a 64-row block, 16 rows empty
    ("bf16", 2, 12, 64, 8, 128, [30, 400]),      # 96 rows: two 64-row blocks, one half empty
    ("bf16", 2, 6, 48, 8, 64, [200, 900]),       # d 64, G 6: 36 rows in one 64-row block
]


@pytest.mark.parametrize("spec", CAUSAL, ids=lambda s: "%s-q%d-%dx%d-d%d" % (s[0], s[2], s[3],
                                                                            s[4], s[5]))
@pytest.mark.parametrize("S", [0, 1, 3])
def test_causal_paged(spec, S):
    dt, B, qlen, hq, hkv, d, lens = spec
    wl = W.make_paged(1200 + qlen * 10 + d, dt, B, qlen, hq, hkv, d, 16, lens, spare_pages=2,
                      outlier_p=0.02)
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=True)
    case("causal paged %s S=%d" % (str(spec), S))
    q, kc, vc = to_dev(wl.q, dt), to_dev(wl.k_cache, dt), to_dev(wl.v_cache, dt)
    out, lse = api.decode_fwd(q, kc, vc, i32_dev(wl.block_table), i32_dev(wl.cache_seqlens),
                              num_splits=S, softmax_scale=wl.scale, max_seqlen_k=wl.max_seqlen_k,
                              causal=True)
    torch.cuda.synchronize()
    e1 = check_out(bits_of(out), ref_o, dt)
    e2 = check_lse(lse.cpu().numpy(), ref_l)
    print("  S=%d max|dO|=%.3g max|dLSE|=%.3g" % (api.last_plan().num_splits, e1, e2), flush=True)


def _append_case(seed, dt, B, qlen, hq, hkv, d, lens, new_len):
    """A workload whose cache already holds L_b + new_len keys; the new rows
    are cut out as k_new/v_new and poisoned in the cache the GPU sees."""
    full = [L + new_len for L in lens]
    wl = W.make_paged(seed, dt, B, qlen, hq, hkv, d, 16, full, spare_pages=2)
    page = wl.page_size
    k_new = np.zeros((B, new_len, hkv, d), dtype=np.uint16)
    v_new = np.zeros_like(k_new)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    nan = {"fp16": 0x7E00, "bf16": 0x7FC0}[dt]
    for b in range(B):
        for t in range(new_len):
            pos = lens[b] + t
            pg, sl = wl.block_table[b, pos // page], pos % page
            k_new[b, t], v_new[b, t] = wl.k_cache[pg, sl], wl.v_cache[pg, sl]
            kc[pg, sl] = nan
            vc[pg, sl] = nan
    return wl, k_new, v_new, kc, vc


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [0, 4])
def test_kv_append_then_attend(causal, S):
    dt, B, qlen, hq, hkv, d, new_len = "bf16", 4, 4, 32, 8, 128, 4
    lens = [0, 13, 500, 1020]
    wl, k_new, v_new, kc_h, vc_h = _append_case(1300 + S, dt, B, qlen, hq, hkv, d, lens, new_len)
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    case("append %d keys then attend, causal=%s S=%d" % (new_len, causal, S))
    kc, vc = to_dev(kc_h, dt), to_dev(vc_h, dt)
    old = i32_dev(np.array(lens, dtype=np.int32))
    out, lse = api.decode_fwd(to_dev(wl.q, dt), kc, vc, i32_dev(wl.block_table), old,
                              num_splits=S, softmax_scale=wl.scale,
                              max_seqlen_k=max(lens) + new_len, k_new=to_dev(k_new, dt),
                              v_new=to_dev(v_new, dt), causal=causal)
    torch.cuda.synchronize()
    check_out(bits_of(out), ref_o, dt)
    check_lse(lse.cpu().numpy(), ref_l)
    # the cache now holds the full workload's bytes, and nothing else changed
    assert np.array_equal(bits_of(kc), wl.k_cache) and np.array_equal(bits_of(vc), wl.v_cache)
    assert np.array_equal(old.cpu().numpy(), np.array(lens, dtype=np.int32))


APPEND_CASES = [
    # name, dtype, B, q_len, Hq, Hkv, d, old lengths, new_len, S, pack_gqa, length sum,
    # causal, appended by the attention kernel itself (None: either)
    ("one key, page edges", "bf16", 8, 1, 32, 8, 128,
     [0, 15, 16, 17, 31, 500, 1023, 1100], 1, 0, -1, False, False, True),
    ("four keys, causal, split edges", "fp16", 6, 4, 16, 4, 128,
     [398, 399, 400, 797, 1195, 3], 4, 3, -1, False, True, True),
    ("head pairs", "fp16", 8, 1, 16, 8, 64, [0, 1, 63, 64, 200, 777, 1500, 2047], 2, 1, -1,
     True, False, True),
    # the compact list's appending copy holds one workgroup per CU against
    # two: a grid of more than 256 workgroups keeps the append kernel
    ("head pairs, compact list", "fp16", 8, 1, 16, 8, 64, [0, 1, 63, 64, 200, 777, 1500, 2047],
     2, 0, -1, True, False, False),
    ("unpacked heads", "bf16", 4, 1, 32, 8, 128, [5, 700, 31, 1024], 3, 2, 0, False, False, True),
    ("two row blocks", "bf16", 2, 4, 64, 2, 128, [600, 95], 4, 0, -1, False, True, True),
    ("head dim 80", "fp16", 4, 1, 8, 2, 80, [14, 300, 0, 999], 1, 0, -1, False, False, True),
    ("head dim 256", "bf16", 4, 2, 8, 4, 256, [30, 1, 640, 257], 3, 2, -1, False, True, True),
    ("five keys: append kernel", "bf16", 4, 1, 32, 8, 128, [14, 300, 0, 999], 5, 0, -1,
     False, False, False),
    ("head dim 32: append kernel", "fp16", 4, 1, 8, 2, 32, [14, 300, 0, 999], 2, 0, -1,
     False, False, False),
    ("compact list", "fp16", 48, 1, 16, 8, 64,
     [int(x) for x in np.random.default_rng(7).integers(1, 3000, 48)], 1, 0, -1, True, False,
     None),
]


@pytest.mark.parametrize("spec", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_kv_append_paths(spec):
    """Appended keys either written by the attention kernel itself (read
    from k_new / v_new, one launch) or by the append kernel first: outputs
    match the oracle on the whole cache, and the cache afterwards holds the
    new rows and nothing else changed."""
    name, dt, B, qlen, hq, hkv, d, lens, new_len, S, pack, use_sum, causal, in_kernel = spec
    wl, k_new, v_new, kc_h, vc_h = _append_case(1400 + len(lens) + d, dt, B, qlen, hq, hkv, d,
                                                lens, new_len)
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    case("append %s: %s B=%d q_len=%d Hq=%d Hkv=%d d=%d new=%d S=%d pack=%d causal=%s"
         % (name, dt, B, qlen, hq, hkv, d, new_len, S, pack, causal))
    kc, vc = to_dev(kc_h, dt), to_dev(vc_h, dt)
    old = i32_dev(np.array(lens, dtype=np.int32))
    total = int(sum(lens)) + B * new_len
    out, lse = api.decode_fwd(to_dev(wl.q, dt), kc, vc, i32_dev(wl.block_table), old,
                              num_splits=S, pack_gqa=pack, softmax_scale=wl.scale,
                              max_seqlen_k=max(lens) + new_len, k_new=to_dev(k_new, dt),
                              v_new=to_dev(v_new, dt), causal=causal,
                              sum_seqlen_k=total if use_sum else None)
    torch.cuda.synchronize()
    plan = api.last_plan()
    print("  plan S=%d heads_per_row=%d extra=%d kernel=%d" % (
        plan.num_splits, plan.heads_per_row, plan.extra_blocks, plan.kernel), flush=True)
    if in_kernel is not None:
        assert (plan.kernel >= 100000) == in_kernel, plan.kernel
    check_out(bits_of(out), ref_o, dt)
    check_lse(lse.cpu().numpy(), ref_l)
    assert np.array_equal(bits_of(kc), wl.k_cache) and np.array_equal(bits_of(vc), wl.v_cache)
    assert np.array_equal(old.cpu().numpy(), np.array(lens, dtype=np.int32))


# ---------------------------------------------------------- ragged splits ----

@pytest.mark.parametrize("lens", [
    [1, 2, 3],                          # every split past the first is empty
    [8192, 1, 1, 1, 1, 1, 1, 1],        # one long sequence, the rest in one split
    [0, 5000, 0, 17, 3000, 1, 2047],    # empty sequences, long and short mixed
    list(range(1, 400, 7)),             # many short sequences, 57 of them
])
@pytest.mark.parametrize("S", [0, 3, 8])
def test_ragged_lengths_with_splits(lens, S):
    """Per-sequence split counts: splits past a sequence's last key skip,
    sequences within one split write directly, the rest merge; the grid runs
    longest first (split-major, and ranked by length when unsplit)."""
    wl = W.make_paged(1500 + len(lens), "fp16", len(lens), 1, 16, 8, 64, 16, lens,
                      spare_pages=2, outlier_p=0.01)
    ref = oracle_paged(wl)
    case("ragged fp16 GQA2 d64, S=%d, lengths %s..." % (S, lens[:8]))
    assert_paged(wl, num_splits=S, ref=ref)
    a, la, _ = run_paged(wl, num_splits=S)
    b, lb, _ = run_paged(wl, num_splits=S)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("spec", [
    ("bf16", 32, 1, 32, 8, 128),   # log-uniform lengths 1..8192, GQA-4 d 128
    ("fp16", 128, 1, 16, 8, 64),   # the same at 128 sequences, GQA-2 d 64
    ("bf16", 32, 8, 32, 8, 128),   # 32 query rows per unit (one 32-row block), causal
])
def test_ragged_batch_with_length_sum_hint(spec):
    """With the sum of the lengths given, the automatic plan splits the
    longest sequences of a ragged batch (S > 1, per-sequence split counts)
    and the result still matches the oracle."""
    dt, B, qlen, hq, hkv, d = spec
    causal = qlen > 1
    wl = W.make_paged(1750 + B + qlen, dt, B, qlen, hq, hkv, d, 16,
                      lambda rng: W.c5_lengths(rng, batch=B), spare_pages=1)
    case("ragged %s B%d q%d Hq%d/Hkv%d d%d with the length-sum hint" % spec)
    q = to_dev(wl.q, dt)
    kc, vc = to_dev(wl.k_cache, dt), to_dev(wl.v_cache, dt)
    bt, sl = i32_dev(wl.block_table), i32_dev(wl.cache_seqlens)
    out, lse = api.decode_fwd(q, kc, vc, bt, sl, softmax_scale=wl.scale,
                              max_seqlen_k=wl.max_seqlen_k, causal=causal,
                              sum_seqlen_k=int(wl.cache_seqlens.sum()))
    torch.cuda.synchronize()
    plan = api.last_plan()
    assert plan.num_splits > 1
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    e1 = check_out(bits_of(out), ref_o, dt, wl.name)
    e2 = check_lse(lse.cpu().numpy(), ref_l)
    print("  plan S=%d grid=%d  max|dO|=%.3g max|dLSE|=%.3g" % (plan.num_splits, plan.grid, e1, e2),
          flush=True)


@pytest.mark.parametrize("S", [257, 1024])
def test_many_splits(S):
    """Up to the largest split count a caller may ask for: 16 keys per split
    at S = 1024, so the fused combine folds 1024 partials (64 batches)."""
    wl = W.make_paged(1650 + S, "bf16", 2, 1, 8, 1, 128, 16, [16384, 9000], spare_pages=1)
    ref = oracle_paged(wl)
    case("many splits: B2 Hq8/Hkv1 d128 L=[16384, 9000], S=%d" % S)
    plan = assert_paged(wl, num_splits=S, ref=ref)
    assert plan.num_splits == S


@pytest.mark.parametrize("B", [1024, 2048])
def test_large_batches(B):
    """The largest batch of the compact split list (1024) and one past it;
    short sequences (under 80 keys), so the split-0 workgroups never rank
    them by length."""
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(0, 80, B)]
    wl = W.make_paged(1600 + B, "bf16", B, 1, 8, 2, 64, 16, lens, spare_pages=2)
    ref = oracle_paged(wl)
    for S in (0, 2):
        case("large batch B=%d GQA4 d64 L<80, S=%d" % (B, S))
        assert_paged(wl, num_splits=S, ref=ref)


# ------------------------------------------------------ compact split list --

COMPACT = [
    # dtype, B, q_len, Hq, Hkv, d, lengths, S, causal, new_len
    ("fp16", 12, 1, 16, 8, 64, [8000, 1, 5, 3000, 0, 17, 1500, 2, 6000, 40, 999, 4000], 5,
     False, 0),
    ("bf16", 9, 1, 32, 8, 128, [5000, 2, 900, 4100, 31, 64, 2500, 7, 3333], 6, False, 0),
    ("bf16", 6, 8, 32, 8, 128, [3000, 10, 2500, 1, 700, 4000], 4, True, 0),  # 32-row blocks
    ("fp16", 5, 8, 64, 8, 64, [2000, 5, 1800, 33, 900], 3, True, 0),         # 64-row blocks
    ("bf16", 4, 4, 32, 8, 128, [1000, 13, 500, 1020], 4, True, 4),           # appended keys
]


@pytest.mark.parametrize("spec", COMPACT, ids=lambda c: "%s-B%d-q%d-d%d-S%d-new%d" % (
    c[0], c[1], c[2], c[5], c[7], c[9]))
def test_compact_split_list(spec):
    """Given a length sum, a split call launches the extra splits from a
    list built on the device instead of every (unit, split) pair.  With the
    right sum each extra workgroup takes one item; with a far smaller one
    (still in range) a single extra workgroup loops over all of them; with a
    larger one some find nothing.  Every run matches the oracle and equals
    the split-major run bit for bit (same splits, same merge order)."""
    dt, B, qlen, hq, hkv, d, lens, S, causal, new_len = spec
    if new_len:
        wl, k_new, v_new, kc_h, vc_h = _append_case(1600 + B, dt, B, qlen, hq, hkv, d, lens,
                                                    new_len)
        attended = [x + new_len for x in lens]
    else:
        wl = W.make_paged(1600 + B, dt, B, qlen, hq, hkv, d, 16, lens, spare_pages=1)
        kc_h, vc_h, k_new, v_new, attended = wl.k_cache, wl.v_cache, None, None, lens
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    q = to_dev(wl.q, dt)
    kc, vc = to_dev(kc_h, dt), to_dev(vc_h, dt)
    bt = i32_dev(wl.block_table)
    sl = i32_dev(np.array(lens, dtype=np.int32))
    kn = to_dev(k_new, dt) if new_len else None
    vn = to_dev(v_new, dt) if new_len else None
    max_len = max(attended)
    true_sum = int(sum(lens))
    results = {}
    for label, hint in (("split-major", None), ("right sum", true_sum), ("sum 1", 1),
                        ("larger sum", min(3 * true_sum, B * max_len))):
        case("compact list %s B%d q%d Hq%d/Hkv%d d%d S=%d causal=%s new=%d, %s" % (
            dt, B, qlen, hq, hkv, d, S, causal, new_len, label))
        out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=S, softmax_scale=wl.scale,
                                  max_seqlen_k=max_len, k_new=kn, v_new=vn, causal=causal,
                                  sum_seqlen_k=hint)
        torch.cuda.synchronize()
        plan = api.last_plan()
        assert plan.num_splits == S
        if hint is None:
            assert plan.extra_blocks == 0 and plan.grid == plan.units * S
        elif plan.extra_blocks > 0:
            assert plan.grid == plan.units + plan.extra_blocks < plan.units * S
        if label in ("right sum", "sum 1"):
            assert plan.extra_blocks > 0
        if label == "sum 1":
            assert plan.extra_blocks == 1
        o, l = bits_of(out), lse.cpu().numpy()
        e1 = check_out(o, ref_o, dt, label)
        e2 = check_lse(l, ref_l)
        print("  extra_blocks=%d grid=%d max|dO|=%.3g max|dLSE|=%.3g" % (
            plan.extra_blocks, plan.grid, e1, e2), flush=True)
        results[label] = (o, l)
    o0, l0 = results["split-major"]
    for label, (o, l) in results.items():
        assert np.array_equal(o, o0) and np.array_equal(l, l0, equal_nan=True), label


RANKED = [
    # dtype, B, Hq, Hkv, d: batches the split-0 workgroups rank by length
    ("bf16", 200, 16, 2, 128),   # not a multiple of 16: padded rank list
    ("fp16", 256, 16, 2, 64),    # the largest ranked batch: four passes of 64 sequences
    ("bf16", 100, 16, 4, 256),   # head dim 256, 4 waves: two passes of 64 sequences
]


@pytest.mark.parametrize("spec", RANKED, ids=lambda c: "%s-B%d-d%d" % (c[0], c[1], c[4]))
def test_ranked_batches_with_ties(spec):
    """Batches of up to 256 sequences with a longest one of at least 1024
    keys and a grid over one round: the split-0 workgroups rank the batch
    (longer first, ties by index), here with many equal lengths.  Every
    sequence must still get its own output."""
    dt, B, hq, hkv, d = spec
    rng = np.random.default_rng(1800 + B)
    lens = [int(x) for x in rng.choice([1, 100, 700, 1024, 1500, 2000], B)]
    lens[0] = 2000
    wl = W.make_paged(1800 + B, dt, B, 1, hq, hkv, d, 16, lens, spare_pages=1)
    ref = oracle_paged(wl)
    for S in (0, 2):
        case("ranked batch %s B%d Hq%d/Hkv%d d%d lengths from 6 values, S=%d" % (
            dt, B, hq, hkv, d, S))
        plan = assert_paged(wl, num_splits=S, ref=ref)
        assert plan.grid > plan.num_cus


@pytest.mark.parametrize("length_sum", [False, True], ids=["split-major", "compact"])
def test_large_ragged_batch_unranked(length_sum):
    """Over 256 sequences the split-0 workgroups keep the batch order (no
    length ranking); a multi-round grid, with and without the compact list."""
    B = 257
    wl = W.make_paged(1700, "fp16", B, 1, 16, 8, 64, 16,
                      lambda rng: W.c5_lengths(rng, batch=B, max_len=3000), spare_pages=1)
    ref = oracle_paged(wl)
    for S in (0, 3):
        case("ragged B%d fp16 GQA-2 d64 up to 3000 keys, S=%d, length sum %s" % (
            B, S, length_sum))
        q, kc, vc = to_dev(wl.q, "fp16"), to_dev(wl.k_cache, "fp16"), to_dev(wl.v_cache, "fp16")
        out, lse = api.decode_fwd(q, kc, vc, i32_dev(wl.block_table), i32_dev(wl.cache_seqlens),
                                  num_splits=S, softmax_scale=wl.scale,
                                  max_seqlen_k=wl.max_seqlen_k,
                                  sum_seqlen_k=int(wl.cache_seqlens.sum()) if length_sum else None)
        torch.cuda.synchronize()
        plan = api.last_plan()
        assert plan.grid > plan.num_cus
        e1 = check_out(bits_of(out), ref[0], "fp16")
        e2 = check_lse(lse.cpu().numpy(), ref[1])
        print("  plan S=%d extra=%d grid=%d max|dO|=%.3g max|dLSE|=%.3g" % (
            plan.num_splits, plan.extra_blocks, plan.grid, e1, e2), flush=True)


GROUPS = [
    # dtype, B, q_len, Hq, Hkv, d, lengths, causal, new_len, page size
    ("fp16", 5, 1, 16, 8, 64, [1, 17, 700, 2000, 64], False, 0, 16),   # G 2: 4 rows per pair
    ("bf16", 4, 1, 32, 4, 64, [300, 1025, 9, 4000], False, 0, 16),     # G 8: 16 rows
    ("bf16", 3, 2, 16, 4, 64, [500, 33, 1800], True, 0, 16),           # q_len 2, causal
    ("fp16", 3, 1, 8, 2, 64, [100, 2047, 5], False, 3, 16),            # keys appended first
    ("bf16", 4, 1, 16, 4, 64, [100, 1500, 47, 999], False, 0, 48),     # 48-key pages
    ("bf16", 4, 1, 16, 4, 32, [1, 900, 3000, 47], False, 0, 16),       # d 32, G 4: a quad
    ("fp16", 3, 2, 16, 8, 32, [700, 2, 1500], True, 0, 16),            # d 32, q_len 2, G 2
    ("fp16", 3, 1, 8, 8, 32, [64, 2500, 33], False, 2, 16),            # d 32 MHA, appended
]


@pytest.mark.parametrize("spec", GROUPS, ids=lambda c: "%s-B%d-q%d-G%d-d%d-new%d-P%d" % (
    c[0], c[1], c[2], c[3] // c[4], c[5], c[8], c[9]))
@pytest.mark.parametrize("S", [1, 3])
def test_head_groups(spec, S):
    """Head dim 64 / 32 with the length sum: a unit is 2 / 4 adjacent KV
    heads on the 128-wide tile, each query row in its head's slice.  The
    output matches the oracle and, bit for bit, the unpacked call (one query
    head per unit on the head dim's own tile): the group only adds exact
    zeros to each score."""
    dt, B, qlen, hq, hkv, d, lens, causal, new_len, page = spec
    R = 128 // d
    if new_len:
        assert page == 16
        wl, k_new, v_new, kc_h, vc_h = _append_case(1900 + B, dt, B, qlen, hq, hkv, d, lens,
                                                    new_len)
        sl_h = np.array(lens, dtype=np.int32)
    else:
        wl = W.make_paged(1900 + B, dt, B, qlen, hq, hkv, d, page, lens, spare_pages=1,
                          outlier_p=0.01)
        kc_h, vc_h, k_new, v_new, sl_h = wl.k_cache, wl.v_cache, None, None, wl.cache_seqlens
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    q = to_dev(wl.q, dt)
    kc, vc = to_dev(kc_h, dt), to_dev(vc_h, dt)
    bt, sl = i32_dev(wl.block_table), i32_dev(sl_h)
    kn = to_dev(k_new, dt) if new_len else None
    vn = to_dev(v_new, dt) if new_len else None
    got = {}
    for pack in ((1, 0) if hq == hkv else (-1, 0)):
        case("head groups %s B%d q%d Hq%d/Hkv%d d%d S=%d causal=%s new=%d pack=%d" % (
            dt, B, qlen, hq, hkv, d, S, causal, new_len, pack))
        out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=S, pack_gqa=pack,
                                  softmax_scale=wl.scale, max_seqlen_k=wl.max_seqlen_k,
                                  k_new=kn, v_new=vn, causal=causal,
                                  sum_seqlen_k=int(wl.cache_seqlens.sum()))
        torch.cuda.synchronize()
        plan = api.last_plan()
        assert plan.heads_per_row == (R if pack != 0 else 1)
        o, l = bits_of(out), lse.cpu().numpy()
        e1 = check_out(o, ref_o, dt)
        e2 = check_lse(l, ref_l)
        print("  heads_per_row=%d units=%d max|dO|=%.3g max|dLSE|=%.3g" % (
            plan.heads_per_row, plan.units, e1, e2), flush=True)
        got[pack] = (o, l)
    grouped = got[1] if hq == hkv else got[-1]
    assert np.array_equal(grouped[0], got[0][0])
    assert np.array_equal(grouped[1], got[0][1], equal_nan=True)


# ------------------------------------------------------------- varlen Q ----

VARLEN = [
    # dtype, Hq, Hkv, d, q lens
    ("bf16", 16, 4, 128, [1, 4, 0, 7, 2]),   # G 4: up to 28 rows (a 32-row block)
    ("fp16", 32, 4, 64, [6, 1, 5, 0, 8]),    # G 8: up to 64 rows (a 64-row block)
    ("fp16", 8, 4, 64, [1, 4, 0, 3, 2]),     # G 2: with the length sum, head pairs (16 rows)
]


@pytest.mark.parametrize("shape", VARLEN, ids=lambda v: "%s-G%d-d%d" % (v[0], v[1] // v[2], v[3]))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,length_sum", [(0, False), (1, False), (3, False), (0, True),
                                          (3, True)])
def test_varlen_queries(shape, causal, S, length_sum):
    """A query count per sequence (cu_seqlens_q), packed; each sequence's
    expected rows come from the oracle run on that sequence alone.  With the
    length sum the planner splits the longest sequence and the call runs the
    compact split list."""
    dt, hq, hkv, d, qlens = shape
    lens = [30, 300, 64, 9, 1000]
    B, maxq = len(lens), max(qlens)
    wl = W.make_paged(1400 + S, dt, B, maxq, hq, hkv, d, 16, lens, spare_pages=2)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    total = int(cu[-1])
    q = np.concatenate([wl.q[b, :qlens[b]] for b in range(B)], axis=0)  # [total, Hq, d]
    ref_o = np.zeros((total, hq, d))
    ref_l = np.full((hq, total), -np.inf)
    for b in range(B):
        if qlens[b] == 0:
            continue
        o, l = oracle.paged_attention(wl.q[b:b + 1, :qlens[b]], wl.k_cache, wl.v_cache,
                                      wl.block_table[b:b + 1], wl.cache_seqlens[b:b + 1], dt,
                                      scale=wl.scale, causal=causal)
        ref_o[cu[b]:cu[b + 1]] = o[0]
        ref_l[:, cu[b]:cu[b + 1]] = l[0]
    case("varlen q_lens %s, causal=%s S=%d length_sum=%s" % (qlens, causal, S, length_sum))
    out, lse = api.decode_varlen_fwd(to_dev(q, dt), to_dev(wl.k_cache, dt), to_dev(wl.v_cache, dt),
                                     i32_dev(wl.block_table), i32_dev(wl.cache_seqlens),
                                     i32_dev(cu), maxq, num_splits=S, softmax_scale=wl.scale,
                                     max_seqlen_k=wl.max_seqlen_k, causal=causal,
                                     sum_seqlen_k=sum(lens) if length_sum else None)
    torch.cuda.synchronize()
    if length_sum:
        plan = api.last_plan()
        print("  plan S=%d extra_blocks=%d heads_per_row=%d" % (
            plan.num_splits, plan.extra_blocks, plan.heads_per_row), flush=True)
        assert plan.extra_blocks > 0
        assert plan.heads_per_row == (2 if (d == 64 and hq // hkv * maxq * 2 <= 16) else 1)
    check_out(bits_of(out), ref_o, dt)
    check_lse(lse.cpu().numpy(), ref_l)
    assert api.last_plan().pack_gqa == 1


# ------------------------------------------------------------- small shapes --

SMALL = [
    # dtype, B, qlen, Hq, Hkv, d, page, lens
    ("bf16", 3, 1, 8, 2, 128, 16, [1, 17, 100]),
    ("fp16", 3, 1, 8, 2, 128, 16, [15, 16, 33]),
    ("bf16", 2, 1, 16, 2, 64, 16, [250, 7]),
    ("fp16", 4, 1, 4, 4, 64, 32, [31, 32, 33, 95]),
    ("bf16", 2, 2, 8, 2, 128, 16, [40, 129]),      # qlen 2, G 4: 8 rows
    ("fp16", 2, 3, 8, 4, 64, 16, [77, 3]),          # 6 rows -> R 8 with 2 idle rows
    ("bf16", 2, 4, 16, 4, 128, 32, [200, 64]),      # 16 rows: one 16-row block
    ("fp16", 1, 8, 8, 1, 128, 16, [300]),           # MQA, 64 rows: one 64-row block
    ("bf16", 5, 1, 8, 8, 128, 16, [1, 2, 3, 16, 17]),  # MHA
    ("fp16", 2, 1, 24, 3, 64, 48, [500, 1000]),     # G 8, page 48
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "%s-B%d-q%d-%dx%d-d%d-p%d" % s[:7])
@pytest.mark.parametrize("S", [0, 1, 2, 5])
def test_small_paged_shapes(spec, S):
    dt, B, qlen, hq, hkv, d, page, lens = spec
    wl = W.make_paged(700 + B * 10 + d + qlen, dt, B, qlen, hq, hkv, d, page, lens,
                      spare_pages=2, outlier_p=0.02)
    case("small paged %s S=%d" % (str(spec), S))
    ref = oracle_paged(wl)
    assert_paged(wl, num_splits=S, ref=ref)
    if S == 1:
        case("small paged %s S=1 pack_gqa=0" % str(spec))
        assert_paged(wl, num_splits=1, pack_gqa=0, ref=ref)


def test_empty_sequences_and_zero_batch():
    wl = W.make_paged(801, "bf16", 4, 1, 8, 2, 128, 16, [0, 20, 0, 1], spare_pages=2)
    for S in (1, 3):
        case("empty sequences (L=0) among others, S=%d" % S)
        out, lse, _ = run_paged(wl, num_splits=S)
        ref_o, ref_l = oracle_paged(wl)
        check_out(out, ref_o, "bf16")
        check_lse(lse, ref_l)
        assert np.all(W.from_bits(out[0], "bf16") == 0) and np.all(np.isneginf(lse[0]))
    case("all sequences empty")
    wl0 = W.make_paged(802, "fp16", 2, 1, 4, 2, 64, 16, [0, 0], spare_pages=1)
    out, lse, _ = run_paged(wl0)
    assert np.all(W.from_bits(out, "fp16") == 0) and np.all(np.isneginf(lse))


def test_partials_and_combine_separately():
    """Rows a9 and a10 on their own: the split kernel's float32 partials
    against the oracle's per-split online recurrence, then the combine
    kernel fed with the oracle's partials."""
    wl = W.make_paged(811, "bf16", 3, 2, 8, 2, 128, 16, [1, 200, 517], spare_pages=2)
    S = 4
    plan = api.decode_plan(3, 2, 8, 2, 128, 16, wl.block_table.shape[1], wl.max_seqlen_k,
                           torch.bfloat16, num_splits=S)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    case("split partials S=4 read back from the workspace")
    out1, lse1, _ = run_paged(wl, num_splits=S, workspace=ws)
    if plan.combine == 2:  # the fused combine leaves its arrival counters at zero
        o_bytes = (S * 48 * 128 * 4 + 255) // 256 * 256 + (S * 48 * 4 + 255) // 256 * 256
        assert int(ws[o_bytes:].view(torch.int32).abs().sum()) == 0
    out2, lse2, _ = run_paged(wl, num_splits=S, workspace=ws)  # same workspace again
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
    nrows = 3 * 2 * 8
    o_gpu, l_gpu = api.workspace_partials(ws, plan, nrows, 128)
    assert plan.split_keys == oracle.split_keys_for(wl.max_seqlen_k, S)
    o_ref, l_ref = oracle.paged_split_partials(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                               wl.cache_seqlens, "bf16", S, plan.split_keys,
                                               block=16, scale=wl.scale)
    o_gpu, l_gpu = o_gpu.cpu().numpy(), l_gpu.cpu().numpy()
    if plan.combine == 2:
        # the fused path writes the partials of splits holding keys of
        # sequences that span two or more splits; the rest add nothing
        C = plan.split_keys
        nsplit = np.maximum(1, -(-wl.cache_seqlens.astype(np.int64) // C))
        seq_of_row = np.arange(nrows) // (2 * 8)  # rows ordered (b, i, hq)
        ns = nsplit[seq_of_row]
        written = (ns[None, :] >= 2) & (np.arange(S)[:, None] < ns[None, :])
        assert written.any() and not written.all()
        # what is skipped: whole sequences within one split, and empty splits
        one_split = np.broadcast_to(ns[None, :] == 1, written.shape)
        assert np.all(one_split[~written] | np.isneginf(l_ref[~written]))
        check_f32(o_gpu[written], o_ref[written])
        check_lse(l_gpu[written], l_ref[written])
    else:
        check_f32(o_gpu, o_ref)
        check_lse(l_gpu, l_ref)
    case("combine kernel on the oracle's partials")
    o32 = o_ref.astype(np.float32)
    l32 = l_ref.astype(np.float32)
    out, lse = api.combine_fwd(torch.from_numpy(o32).cuda(), torch.from_numpy(l32).cuda(), 3, 2,
                               8, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.combine(o32.astype(np.float64), l32.astype(np.float64))
    check_out(bits_of(out).reshape(nrows, 128), ref_o, "bf16")
    check_lse(lse.cpu().numpy().transpose(0, 2, 1).reshape(nrows), ref_l)


@pytest.mark.parametrize("d", [1, 5, 64, 200, 512])
def test_combine_any_head_dim(d):
    rng = np.random.default_rng(d)
    S, B, qlen, H = 5, 2, 3, 4
    n = B * qlen * H
    o = rng.standard_normal((S, n, d)).astype(np.float32)
    l = (3 * rng.standard_normal((S, n))).astype(np.float32)
    l[1, :4] = -np.inf
    l[:, 5] = -np.inf  # row 5: every partial empty
    o[:, 5] = 0
    case("combine S=5 head_dim=%d" % d)
    out, lse = api.combine_fwd(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), B, qlen,
                               H, dtype=torch.float16)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.combine(o.astype(np.float64), l.astype(np.float64))
    check_out(bits_of(out).reshape(n, d), ref_o, "fp16")
    check_lse(lse.cpu().numpy().transpose(0, 2, 1).reshape(n), ref_l)


def test_bitwise_determinism_and_page_permutation():
    wl = W.make_paged(821, "bf16", 4, 1, 32, 8, 128, 16, [300, 1000, 17, 640], spare_pages=3)
    case("determinism: two runs bitwise equal, S=1 and S=4")
    for S in (1, 4):
        a, la, _ = run_paged(wl, num_splits=S)
        b, lb, _ = run_paged(wl, num_splits=S)
        assert np.array_equal(a, b) and np.array_equal(la, lb)
    case("physical page permutation leaves the output bitwise unchanged")
    rng = np.random.default_rng(5)
    n = wl.k_cache.shape[0]
    perm = rng.permutation(n)
    kc = np.empty_like(wl.k_cache); vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache; vc[perm] = wl.v_cache
    wl2 = W.PagedWorkload(**{**wl.__dict__, "k_cache": kc, "v_cache": vc,
                             "block_table": perm[wl.block_table].astype(np.int32)})
    for S in (1, 4):
        a, la, _ = run_paged(wl, num_splits=S)
        b, lb, _ = run_paged(wl2, num_splits=S)
        assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_fused_combine_soak():
    """Bounded soak of the fused combine (partials written through, the
    arrival atomic, the last split's merge): 240 seeded split calls over 12
    ragged shapes, each call repeated on a workspace shared by every call of
    its shape, and with the compact list, and compared bit for bit with a
    first split-major run.  A stale partial or a counter not rearmed would
    change some output; the test stops at the first mismatch."""
    rng = np.random.default_rng(4242)
    shapes = []
    for k in range(12):
        dt = ("bf16", "fp16")[k % 2]
        d = (128, 64, 128, 256)[k % 4]
        hkv = (8, 4, 2, 8)[k % 4]
        G = (4, 2, 8, 1)[k % 4]
        B = int(rng.integers(2, 24))
        lens = [int(x) for x in rng.integers(0, 6000, B)]
        lens[0] = 6000
        S = int(rng.integers(2, 17))
        shapes.append((dt, B, hkv * G, hkv, d, lens, S))
    calls = 0
    for k, (dt, B, hq, hkv, d, lens, S) in enumerate(shapes):
        wl = W.make_paged(4300 + k, dt, B, 1, hq, hkv, d, 16, lens, spare_pages=1)
        q, kc, vc = to_dev(wl.q, dt), to_dev(wl.k_cache, dt), to_dev(wl.v_cache, dt)
        bt, sl = i32_dev(wl.block_table), i32_dev(wl.cache_seqlens)
        case("soak %d: %s B%d Hq%d/Hkv%d d%d S=%d, 20 calls" % (k, dt, B, hq, hkv, d, S))
        ref, ref_l = None, None
        ws = {}
        for rep in range(20):
            hint = int(sum(lens)) if rep % 2 else None
            key = hint is not None
            out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=S, softmax_scale=wl.scale,
                                      max_seqlen_k=wl.max_seqlen_k, sum_seqlen_k=hint,
                                      workspace=ws.get(key))
            if key not in ws:
                plan = api.last_plan()
                ws[key] = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
            o, l = bits_of(out), lse.cpu().numpy()
            if ref is None:
                ref, ref_l = o, l
                ro, rl = oracle_paged(wl)
                check_out(o, ro, dt, "soak %d" % k)
                check_lse(l, rl)
            else:
                assert np.array_equal(o, ref), "soak %d call %d: output differs" % (k, rep)
                assert np.array_equal(l.view(np.uint32), ref_l.view(np.uint32)), (k, rep)
            calls += 1
    print("  %d split calls, all bitwise equal to the first run of their shape" % calls, flush=True)


@pytest.mark.parametrize("q_len,G,d,length_sum", [(1, 4, 128, False), (1, 2, 64, True),
                                                  (4, 8, 128, False), (8, 8, 128, True),
                                                  (8, 4, 64, False), (2, 4, 256, False)],
                         ids=["rows4", "pairs-compact", "rows32", "rows64-compact", "rows32-d64",
                              "d256"])
def test_split_calls_repeat_on_one_workspace(q_len, G, d, length_sum):
    """Split calls with one, two and four 16-row blocks per workgroup, with
    and without the compact list, twice on one workspace: the arrival
    counters are zero after each call, the second output is the first bit
    for bit, and both are within the bar of the oracle."""
    hkv = 2
    lens = [900, 5, 2100, 1300, 0]
    wl = W.make_paged(5100 + q_len * 10 + d, "bf16", len(lens), q_len, hkv * G, hkv, d, 16, lens,
                      spare_pages=1)
    q, kc, vc = to_dev(wl.q, "bf16"), to_dev(wl.k_cache, "bf16"), to_dev(wl.v_cache, "bf16")
    bt, sl = i32_dev(wl.block_table), i32_dev(wl.cache_seqlens)
    hint = int(sum(lens)) if length_sum else None
    case("split calls on one workspace: q_len %d G %d d %d, length sum %s"
         % (q_len, G, d, length_sum))
    plan = api.decode_plan(len(lens), q_len, hkv * G, hkv, d, 16, wl.block_table.shape[1],
                           wl.max_seqlen_k, torch.bfloat16, num_splits=3, sum_seqlen_k=hint or 0)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    nrows = len(lens) * q_len * hkv * G
    c0 = (3 * nrows * d * 4 + 255) // 256 * 256 + (3 * nrows * 4 + 255) // 256 * 256
    res = []
    for _ in range(2):
        out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=3, softmax_scale=wl.scale,
                                  max_seqlen_k=wl.max_seqlen_k, sum_seqlen_k=hint, workspace=ws)
        torch.cuda.synchronize()
        assert int((ws[c0:] != 0).sum()) == 0, "arrival counters not rearmed"
        res.append((bits_of(out), lse.cpu().numpy()))
    assert api.last_plan().num_splits == 3
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1].view(np.uint32), res[1][1].view(np.uint32))
    ro, rl = oracle_paged(wl)
    check_out(res[0][0], ro, "bf16", "split calls on one workspace")
    check_lse(res[0][1], rl)


@pytest.mark.parametrize("dt,B,hkv,G,d,length_sum,pack", [
    ("bf16", 3, 8, 4, 128, False, -1),   # full groups of one sequence's 8 KV heads
    ("bf16", 5, 4, 8, 128, False, -1),   # groups spanning two sequences, a short last group
    ("fp16", 4, 8, 2, 64, False, -1),    # 128-byte slices
    ("fp16", 3, 16, 1, 64, False, -1),   # G = 1, 16 KV heads
    ("fp16", 6, 8, 2, 64, True, -1),     # head pairs (256-byte group slices), compact list
    ("bf16", 3, 8, 4, 128, False, 0),    # unpacked: units are query heads, no reordering
], ids=["d128-h8", "d128-h4", "d64-h8", "d64-h16-mha", "pairs", "unpacked"])
def test_xcd_order_of_units(dt, B, hkv, G, d, length_sum, pack):
    """Head units reordered by XCD within groups of 8 workgroups: every unit
    is computed exactly once (each output row against the oracle), with
    and without splits."""
    lens = [int(x) for x in np.random.default_rng(B * 100 + d + hkv).integers(1, 2500, B)]
    wl = W.make_paged(6100 + B + d + hkv, dt, B, 1, hkv * G, hkv, d, 16, lens, spare_pages=1)
    ro, rl = oracle_paged(wl)
    for S in (1, 3):
        case("XCD order: %s B%d Hkv%d G%d d%d sum %s pack %d S=%d" % (dt, B, hkv, G, d, length_sum,
                                                                   pack, S))
        out, lse, plan = run_paged(wl, num_splits=S, pack_gqa=pack, sum_hint=length_sum)
        check_out(out, ro, dt, "XCD order", strict=True)
        check_lse(lse, rl)


@pytest.mark.parametrize("length_sum,d", [(False, 128), (True, 128), (True, 64)],
                         ids=["split-major", "compact", "compact-head-pairs"])
def test_hip_graph_replays_match_eager(length_sum, d):
    """A split call (fused combine, arrival counters rearmed by the kernel,
    no memset) captured in a HIP graph and replayed, with eager calls on
    other inputs in between: every replay equals the eager result.  With
    the length sum the call launches the compact split list (and at head
    dim 64 reads head pairs)."""
    wl = W.make_paged(1800, "bf16", 4, 2, 16, 4, d, 16, [700, 33, 1500, 1], spare_pages=2)
    q, kc, vc = to_dev(wl.q, "bf16"), to_dev(wl.k_cache, "bf16"), to_dev(wl.v_cache, "bf16")
    bt, sl = i32_dev(wl.block_table), i32_dev(wl.cache_seqlens)
    q2 = to_dev(W.make_paged(1801, "bf16", 4, 2, 16, 4, d, 16, [700, 33, 1500, 1]).q, "bf16")
    hint = int(wl.cache_seqlens.sum()) if length_sum else None
    case("HIP graph capture of a 4-split decode call, d %d, 5 replays, length sum %s"
         % (d, hint))
    call = api.PreparedDecode(q, kc, vc, bt, sl, num_splits=4, softmax_scale=wl.scale,
                              max_seqlen_k=wl.max_seqlen_k, sum_seqlen_k=hint)
    other = api.PreparedDecode(q2, kc, vc, bt, sl, num_splits=4, softmax_scale=wl.scale,
                               max_seqlen_k=wl.max_seqlen_k, sum_seqlen_k=hint)
    call()
    torch.cuda.synchronize()
    assert (api.last_plan().extra_blocks > 0) == length_sum
    assert api.last_plan().heads_per_row == (2 if (length_sum and d == 64) else 1)
    ref_o, ref_l = bits_of(call.out).copy(), call.lse.cpu().numpy().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the side stream, as graph capture wants
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    graph_call = api.PreparedDecode(q, kc, vc, bt, sl, num_splits=4, softmax_scale=wl.scale,
                                    max_seqlen_k=wl.max_seqlen_k, out=call.out, lse=call.lse,
                                    workspace=call.workspace, stream=None, sum_seqlen_k=hint)
    with torch.cuda.graph(g):
        graph_call.args[-1] = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        graph_call()
    for rep in range(5):
        call.out.zero_()
        other()  # eager work on the same workspace shape, other queries
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(call.out), ref_o), "replay %d" % rep
        assert np.array_equal(call.lse.cpu().numpy(), ref_l), "replay %d" % rep


@pytest.mark.parametrize("new_len", [1, 5])
def test_hip_graph_replays_with_appended_keys(new_len):
    """A 4-split kvcache call (new keys written by the attention launch
    itself with 1 key a sequence, by the append kernel first with 5)
    captured in a HIP graph: before each replay the new rows are poisoned
    again in the cache; every replay writes them back and equals the eager
    result."""
    dt = "bf16"
    wl, k_new, v_new, kc_h, vc_h = _append_case(1850 + new_len, dt, 4, 1, 32, 8, 128,
                                                [700, 33, 1500, 1], new_len)
    q = to_dev(wl.q, dt)
    kc, vc = to_dev(kc_h, dt), to_dev(vc_h, dt)
    kc0, vc0 = kc.clone(), vc.clone()
    bt, old = i32_dev(wl.block_table), i32_dev(np.array([700, 33, 1500, 1], dtype=np.int32))
    kn, vn = to_dev(k_new, dt), to_dev(v_new, dt)
    case("HIP graph capture of a 4-split kvcache call, %d new keys, 5 replays" % new_len)
    mk = lambda **kw: api.PreparedDecode(q, kc, vc, bt, old, num_splits=4,
                                         softmax_scale=wl.scale, max_seqlen_k=1500 + new_len,
                                         k_new=kn, v_new=vn, **kw)
    call = mk()
    call()
    torch.cuda.synchronize()
    assert (api.last_plan().kernel >= 100000) == (new_len == 1)
    ref_o, ref_l = bits_of(call.out).copy(), call.lse.cpu().numpy().copy()
    assert np.array_equal(bits_of(kc), wl.k_cache) and np.array_equal(bits_of(vc), wl.v_cache)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the side stream, as graph capture wants
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    graph_call = mk(out=call.out, lse=call.lse, workspace=call.workspace)
    with torch.cuda.graph(g):
        graph_call.args[-1] = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        graph_call()
    for rep in range(5):
        call.out.zero_()
        kc.copy_(kc0)
        vc.copy_(vc0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(call.out), ref_o), "replay %d" % rep
        assert np.array_equal(call.lse.cpu().numpy(), ref_l), "replay %d" % rep
        assert np.array_equal(bits_of(kc), wl.k_cache), "replay %d" % rep
        assert np.array_equal(bits_of(vc), wl.v_cache), "replay %d" % rep


def test_side_stream_split_call():
    """A split call on a stream other than torch's current one: the binding
    allocates the outputs and zero-fills the workspace (the fused combine's
    arrival counters) on that stream, so the fill is ordered before the
    kernel; two calls in a row, each with a fresh workspace."""
    wl = W.make_paged(1960, "bf16", 3, 1, 16, 4, 128, 16, [3000, 17, 2200], spare_pages=1)
    ref_o, ref_l = oracle_paged(wl)
    q, kc, vc = to_dev(wl.q, "bf16"), to_dev(wl.k_cache, "bf16"), to_dev(wl.v_cache, "bf16")
    bt, sl = i32_dev(wl.block_table), i32_dev(wl.cache_seqlens)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(2):
        case("side stream: paged bf16 B3 Hq16/Hkv4 d128, S=4, call %d" % rep)
        out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=4, softmax_scale=wl.scale,
                                  max_seqlen_k=wl.max_seqlen_k, stream=side)
        side.synchronize()
        assert api.last_plan().num_splits == 4
        check_out(bits_of(out), ref_o, "bf16", strict=True)
        check_lse(lse.cpu().numpy(), ref_l)


def test_last_plan_matches_host_plan():
    wl = W.c4_long()
    case("last_plan after a forward equals the host plan (long context, planner)")
    run_paged(wl)
    got = api.last_plan().as_dict()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = api.decode_plan(4, 1, 32, 4, 128, 16, wl.block_table.shape[1], wl.max_seqlen_k,
                           torch.bfloat16, num_cus=cus).as_dict()
    assert got == want
    print("  device CUs=%d plan=%s" % (cus, got), flush=True)


def test_workspace_too_small_is_rejected_and_writes_nothing():
    wl = W.make_paged(831, "fp16", 2, 1, 8, 2, 64, 16, [100, 200], spare_pages=1)
    q = to_dev(wl.q, "fp16")
    out = torch.full_like(q, 7.0)
    ws = torch.zeros(64, dtype=torch.uint8, device="cuda")
    case("workspace too small for S=3")
    with pytest.raises(Exception) as ei:
        api.decode_fwd(q, to_dev(wl.k_cache, "fp16"), to_dev(wl.v_cache, "fp16"),
                       i32_dev(wl.block_table), i32_dev(wl.cache_seqlens), num_splits=3,
                       out=out, workspace=ws)
    assert "ATTN_ERR_WORKSPACE" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_scale_override():
    wl = W.make_paged(841, "bf16", 2, 1, 8, 2, 128, 16, [60, 90], spare_pages=1, scale=0.37)
    case("softmax_scale=0.37")
    assert_paged(wl)


# --------------------------------------------------------- seeded mixtures --

def _random_config(k):
    """Configuration k of a fixed, seeded mixture over dtype, head dim (with
    padded and element-load dims), GQA, q_len, causal, batch, log-uniform
    lengths, outlier rows and split count."""
    rng = np.random.default_rng(9000 + k)
    dt = ["bf16", "fp16"][rng.integers(2)]
    d = int(rng.choice([32, 64, 80, 96, 100, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    qlen = int(rng.choice([1, 1, 2, 4, 8]))
    causal = bool(qlen > 1 and rng.integers(2))
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in np.exp(rng.uniform(0, np.log(3000), B)).astype(int)]
    outl = float(rng.choice([0.0, 0.01, 0.05]))
    S = int(rng.choice([0, 1, 3, 8]))
    return dt, d, hkv, G, qlen, causal, B, lens, outl, S


@pytest.mark.parametrize("k", range(24))
def test_seeded_mixture(k):
    dt, d, hkv, G, qlen, causal, B, lens, outl, S = _random_config(k)
    wl = W.make_paged(9100 + k, dt, B, qlen, hkv * G, hkv, d, 16, lens, spare_pages=1,
                      outlier_p=outl)
    case("mixture %d: %s d%d Hkv%d G%d q%d causal=%s B%d L=%s outliers=%g S=%d"
         % (k, dt, d, hkv, G, qlen, causal, B, lens, outl, S))
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    out, lse = api.decode_fwd(to_dev(wl.q, dt), to_dev(wl.k_cache, dt), to_dev(wl.v_cache, dt),
                              i32_dev(wl.block_table), i32_dev(wl.cache_seqlens), num_splits=S,
                              softmax_scale=wl.scale, max_seqlen_k=max(wl.max_seqlen_k, 0),
                              causal=causal)
    torch.cuda.synchronize()
    check_out(bits_of(out), ref_o, dt)
    check_lse(lse.cpu().numpy(), ref_l)


@pytest.mark.parametrize("k", range(24, 48))
def test_seeded_mixture_with_length_sum(k):
    """More of the seeded mixture, each call given its length sum, so the
    plans also use the ragged split rule, the compact split list and head
    groups where they apply (every other configuration takes head dim 32 or
    64, where head groups exist)."""
    dt, d, hkv, G, qlen, causal, B, lens, outl, S = _random_config(k)
    if k % 2 == 0:
        d = (32, 64)[(k // 2) % 2]
    wl = W.make_paged(9100 + k, dt, B, qlen, hkv * G, hkv, d, 16, lens, spare_pages=1,
                      outlier_p=outl)
    case("mixture %d with the length sum: %s d%d Hkv%d G%d q%d causal=%s B%d L=%s "
         "outliers=%g S=%d" % (k, dt, d, hkv, G, qlen, causal, B, lens, outl, S))
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    out, lse = api.decode_fwd(to_dev(wl.q, dt), to_dev(wl.k_cache, dt), to_dev(wl.v_cache, dt),
                              i32_dev(wl.block_table), i32_dev(wl.cache_seqlens), num_splits=S,
                              softmax_scale=wl.scale, max_seqlen_k=max(wl.max_seqlen_k, 0),
                              causal=causal, sum_seqlen_k=int(sum(lens)))
    torch.cuda.synchronize()
    plan = api.last_plan()
    e1 = check_out(bits_of(out), ref_o, dt)
    e2 = check_lse(lse.cpu().numpy(), ref_l)
    print("  plan S=%d heads_per_row=%d extra_blocks=%d max|dO|=%.3g max|dLSE|=%.3g" % (
        plan.num_splits, plan.heads_per_row, plan.extra_blocks, e1, e2), flush=True)


@pytest.mark.parametrize("k", range(48, 72))
def test_seeded_mixture_with_appends(k):
    """More of the seeded mixture as kvcache calls: 1 to 5 new keys a
    sequence (written by the attention launch itself or by the append kernel
    first, whichever the call takes), the length sum on every other call.
    Outputs match the oracle over the whole cache and the cache afterwards
    holds the new rows, byte for byte."""
    dt, d, hkv, G, qlen, causal, B, lens, _, S = _random_config(k)
    new_len = 1 + k % 5
    wl, k_new, v_new, kc_h, vc_h = _append_case(9200 + k, dt, B, qlen, hkv * G, hkv, d, lens,
                                                new_len)
    case("mixture %d with %d new keys: %s d%d Hkv%d G%d q%d causal=%s B%d L=%s S=%d"
         % (k, new_len, dt, d, hkv, G, qlen, causal, B, lens, S))
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, dt, scale=wl.scale, causal=causal)
    kc, vc = to_dev(kc_h, dt), to_dev(vc_h, dt)
    total = int(sum(lens)) + B * new_len
    out, lse = api.decode_fwd(to_dev(wl.q, dt), kc, vc, i32_dev(wl.block_table),
                              i32_dev(np.array(lens, dtype=np.int32)), num_splits=S,
                              softmax_scale=wl.scale, max_seqlen_k=max(lens) + new_len,
                              k_new=to_dev(k_new, dt), v_new=to_dev(v_new, dt), causal=causal,
                              sum_seqlen_k=total if k % 2 else None)
    torch.cuda.synchronize()
    plan = api.last_plan()
    e1 = check_out(bits_of(out), ref_o, dt)
    e2 = check_lse(lse.cpu().numpy(), ref_l)
    print("  plan S=%d heads_per_row=%d extra_blocks=%d kernel=%d max|dO|=%.3g max|dLSE|=%.3g"
          % (plan.num_splits, plan.heads_per_row, plan.extra_blocks, plan.kernel, e1, e2),
          flush=True)
    assert np.array_equal(bits_of(kc), wl.k_cache) and np.array_equal(bits_of(vc), wl.v_cache)
