"""Host-only checks of the C-ABI library: it loads, exports every symbol the
header declares, plans like the oracle planner, and rejects bad arguments
before touching any device (no compute call is made here)."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

from oracle import planner as oplan
from split_kv_paged_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from split_kv_paged_amd import build
        build.build()
    return L.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    declared = header_functions()
    assert set(declared) == set(L.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    out = os.popen("nm -D --defined-only %s" % L.LIB_PATH).read()
    for name in declared:
        assert re.search(r"\bT %s\b" % name, out), name


def test_abi_version(lib):
    text = open(HEADER).read()
    v = int(re.search(r"#define ATTN_ABI_VERSION (\d+)", text).group(1))
    assert lib.attn_abi_version() == v


def test_status_strings(lib):
    for code in L.STATUS:
        assert lib.attn_status_str(code)
    assert lib.attn_status_str(99) == b"unknown status"


def _plan(lib, **kw):
    shape = L.DecodeShape(kw["batch"], kw["q_len"], kw["hq"], kw["hkv"], kw.get("d", 128),
                          kw.get("page", 16), kw.get("maxp", 64), kw["max_L"], kw.get("dt", 1),
                          kw.get("sum_L", 0))
    plan = L.Plan()
    code = lib.attn_decode_plan(ctypes.byref(shape), kw.get("S", 0), kw.get("pack", -1),
                                kw.get("cus", 0), ctypes.byref(plan))
    return code, plan


PLAN_GRID = list(itertools.product([1, 2, 3, 4, 7, 13, 32, 128], [1, 2, 4, 8], [1, 2, 3, 4, 8],
                                   [1, 2, 4, 8], [1, 100, 513, 1024, 4096, 16384],
                                   [0, 1, 4], [-1, 0, 1]))


def wg_rows(rows):
    """Packed rows one workgroup carries at head dims 64 and 128 (16, 32 or
    64): the unit tile of the split rule."""
    return 16 if rows <= 16 else 32 if rows <= 32 else 64


def unit_tile(q_len, G, pack):
    packed = oplan.should_pack_gqa(False, q_len, G, 16) if pack < 0 else bool(pack)
    return wg_rows(q_len * G if packed else q_len)


def test_plan_matches_oracle_planner(lib):
    """Bit-exact parity of the host planning step with the oracle planner,
    over a grid of batch x qLen x G x Hkv x max_seqlen_k x splits x pack."""
    n = 0
    for batch, q_len, G, hkv, max_L, S, pack in PLAN_GRID:
        hq = G * hkv
        maxp = (max_L + 15) // 16
        code, plan = _plan(lib, batch=batch, q_len=q_len, hq=hq, hkv=hkv, max_L=max_L,
                           maxp=maxp, S=S, pack=pack)
        assert code == 0
        want = oplan.plan(batch, q_len, hq, hkv, max_L, 256, 16, 128, S, pack,
                          unit_block_m=unit_tile(q_len, G, pack))
        assert (plan.num_splits, bool(plan.pack_gqa)) == want, (batch, q_len, G, hkv, max_L, S,
                                                                 pack)
        n += 1
    assert n == len(PLAN_GRID)


@pytest.mark.parametrize("cus", [80, 132, 304])
def test_plan_uses_given_cu_count(lib, cus):
    for batch, hkv, max_L in [(1, 1, 8192), (2, 4, 16384), (5, 8, 3000), (64, 8, 1024)]:
        code, plan = _plan(lib, batch=batch, q_len=1, hq=4 * hkv, hkv=hkv, max_L=max_L,
                           maxp=(max_L + 15) // 16, cus=cus)
        assert code == 0
        assert plan.num_cus == cus
        assert (plan.num_splits, bool(plan.pack_gqa)) == oplan.plan(batch, 1, 4 * hkv, hkv,
                                                                    max_L, cus, 16, 128, 0, -1)


def test_plan_fields_are_consistent(lib):
    code, plan = _plan(lib, batch=4, q_len=1, hq=32, hkv=4, max_L=16384, maxp=1024)
    assert code == 0
    assert plan.num_splits == 14 and plan.pack_gqa == 1
    assert plan.rows_per_unit == 8 and plan.rows_per_block == 16 and plan.row_blocks == 1
    assert plan.units == 4 * 4 and plan.grid == 16 * 14 and plan.combine == 2
    assert plan.split_keys == 16 * 74  # ceil(1024 granules / 14) = 74
    nrows = 4 * 1 * 32
    o = (14 * nrows * 128 * 4 + 255) // 256 * 256
    # + 16 arrival counters, one per 128-byte line
    assert plan.workspace_bytes == o + (14 * nrows * 4 + 255) // 256 * 256 + 16 * 128
    # the target paged decode workload: packed, one split, no workspace
    code, plan = _plan(lib, batch=32, q_len=1, hq=32, hkv=8, max_L=1100, maxp=69)
    assert (plan.num_splits, plan.pack_gqa, plan.rows_per_block, plan.grid) == (1, 1, 16, 256)
    assert plan.workspace_bytes == 0 and plan.combine == 0
    # rows beyond 16 go to row blocks
    code, plan = _plan(lib, batch=2, q_len=3, hq=32, hkv=4, max_L=512, maxp=32, S=1, pack=1)
    assert plan.rows_per_unit == 24 and plan.rows_per_block == 32 and plan.row_blocks == 1
    # beyond 32 rows: 64-row blocks (d 64 and 128)
    code, plan = _plan(lib, batch=2, q_len=8, hq=64, hkv=8, max_L=512, maxp=32, S=1, pack=1, d=64)
    assert plan.rows_per_unit == 64 and plan.rows_per_block == 64 and plan.row_blocks == 1
    code, plan = _plan(lib, batch=2, q_len=5, hq=8, hkv=1, max_L=512, maxp=32, S=1, pack=1, d=64)
    assert plan.rows_per_unit == 40 and plan.rows_per_block == 64 and plan.row_blocks == 1
    code, plan = _plan(lib, batch=2, q_len=8, hq=64, hkv=8, max_L=512, maxp=32, S=1, pack=1)
    assert plan.rows_per_unit == 64 and plan.rows_per_block == 64 and plan.row_blocks == 1
    code, plan = _plan(lib, batch=2, q_len=12, hq=64, hkv=8, max_L=512, maxp=32, S=1, pack=1)
    assert plan.rows_per_unit == 96 and plan.rows_per_block == 64 and plan.row_blocks == 2
    assert plan.units == 2 * 8 * 2 and plan.grid == plan.units
    # two 16-row blocks per workgroup only where that kernel exists (d 64/128)
    code, plan = _plan(lib, batch=2, q_len=3, hq=32, hkv=4, max_L=512, maxp=32, S=1, pack=1,
                       d=96)
    assert plan.rows_per_block == 16 and plan.row_blocks == 2
    # unpacked: one query head per unit
    code, plan = _plan(lib, batch=2, q_len=2, hq=8, hkv=2, max_L=512, maxp=32, S=1, pack=0)
    assert plan.rows_per_unit == 2 and plan.units == 2 * 8


@pytest.mark.parametrize("kw,per_row", [
    (dict(q_len=1, hq=8, hkv=2), 2),     # d 64, G 4: 8 rows per pair
    (dict(q_len=2, hq=8, hkv=2), 2),     # 16 rows per pair: still one block
    (dict(q_len=3, hq=8, hkv=2), 1),     # 24 rows: no pair
    (dict(q_len=1, hq=16, hkv=2), 2),    # G 8: 16 rows
    (dict(q_len=1, hq=32, hkv=2), 1),    # G 16: 32 rows
    (dict(q_len=1, hq=6, hkv=3), 1),     # an odd number of KV heads
    (dict(q_len=1, hq=8, hkv=8), 2),     # MHA decode: the rule's no-pack changes no row
    (dict(q_len=1, hq=8, hkv=8, pack=0), 1),  # unless packing is refused explicitly
    (dict(q_len=1, hq=8, hkv=2, pack=0), 1),
    (dict(q_len=1, hq=8, hkv=2, d=128), 1),
    (dict(q_len=1, hq=8, hkv=2, d=96), 1),
    (dict(q_len=1, hq=16, hkv=4, d=32), 4),   # d 32, G 4: 16 rows per quad
    (dict(q_len=1, hq=8, hkv=8, d=32, pack=1), 4),  # MHA packed: 4 rows per quad
    (dict(q_len=1, hq=24, hkv=4, d=32), 1),   # G 6: 24 rows per quad
    (dict(q_len=1, hq=12, hkv=6, d=32), 1),   # 6 KV heads: not a multiple of 4
    (dict(q_len=2, hq=8, hkv=4, d=32), 4),    # q_len 2, G 2: 16 rows
])
def test_head_group_plan(lib, kw, per_row):
    """Paged head dim 64 / 32 with the length sum: 2 / 4 adjacent KV heads
    per unit when the group's packed rows fit one 16-row block; units, rows
    and the split rule then count groups.  Without the sum, no groups."""
    kw = dict(kw)
    d = kw.pop("d", 64)
    code, plan = _plan(lib, batch=3, max_L=512, maxp=32, d=d, **kw)
    assert code == 0 and plan.heads_per_row == 1
    code, plan = _plan(lib, batch=3, max_L=512, maxp=32, d=d, sum_L=1200, **kw)
    assert code == 0 and plan.heads_per_row == per_row
    G = kw["hq"] // kw["hkv"]
    if per_row > 1:
        assert plan.pack_gqa == 1 and plan.rows_per_unit == kw["q_len"] * per_row * G
        assert plan.units == 3 * (kw["hkv"] // per_row) and plan.kernel == 41128
        assert plan.rows_per_block == 16 and plan.row_blocks == 1
        # the split rule sees the groups: the pages' rule with Hkv / R and R G
        want = oplan.plan(3, kw["q_len"], kw["hq"], kw["hkv"] // per_row, 512, 256, 16, 128,
                          0, kw.get("pack", -1))
        assert plan.num_splits == want[0]
    # the workspace holds head_dim-wide partials of the real query rows
    code, plan = _plan(lib, batch=3, max_L=4096, maxp=256, d=d, S=3, sum_L=9000, **kw)
    nrows = 3 * kw["q_len"] * kw["hq"]
    o = (3 * nrows * d * 4 + 255) // 256 * 256
    assert plan.workspace_bytes == o + (3 * nrows * 4 + 255) // 256 * 256 + (
        (plan.units * 128 + 255) // 256 * 256)


def test_plan_kernel_ids_name_the_tile_and_load_path(lib):
    for d, want in [(64, 11064), (128, 11128), (32, 11032), (256, 11256), (96, 21128),
                    (1, 31032), (200, 21256), (33, 31064), (16, 21032), (130, 31256)]:
        code, plan = _plan(lib, batch=2, q_len=1, hq=8, hkv=2, max_L=512, maxp=32, d=d)
        assert code == 0 and plan.kernel == want, (d, plan.kernel)
    # with the length sum, d 64 with two KV heads: a head group on the 128-wide tile
    code, plan = _plan(lib, batch=2, q_len=1, hq=8, hkv=2, max_L=512, maxp=32, d=64, sum_L=900)
    assert code == 0 and plan.kernel == 41128 and plan.heads_per_row == 2
    code, plan = _plan(lib, batch=2, q_len=1, hq=4, hkv=1, max_L=512, maxp=32, d=64, sum_L=900)
    assert code == 0 and plan.kernel == 11064 and plan.heads_per_row == 1  # one KV head
    shape = L.DenseShape(8, 2, 1, 512, 80, 0)
    plan = L.Plan()
    assert lib.attn_dense_plan(ctypes.byref(shape), 0, 0, ctypes.byref(plan)) == 0
    assert plan.kernel == 20128  # 80: a multiple of 8, 16-byte loads with a column mask


@pytest.mark.parametrize("field,value,want", [
    ("batch", -1, "ATTN_ERR_SHAPE"), ("q_len", 0, "ATTN_ERR_SHAPE"),
    ("hq", 0, "ATTN_ERR_SHAPE"), ("hkv", 3, "ATTN_ERR_SHAPE"),
    ("d", 257, "ATTN_ERR_UNSUPPORTED"), ("d", 0, "ATTN_ERR_SHAPE"),
    ("page", 0, "ATTN_ERR_SHAPE"), ("page", 8, "ATTN_ERR_UNSUPPORTED"),
    ("maxp", 0, "ATTN_ERR_SHAPE"), ("max_L", 8193, "ATTN_ERR_SHAPE"),
    ("max_L", -5, "ATTN_ERR_SHAPE"), ("dt", 2, "ATTN_ERR_UNSUPPORTED"),
    ("S", -1, "ATTN_ERR_ARG"), ("S", 1025, "ATTN_ERR_ARG"), ("pack", 2, "ATTN_ERR_ARG"),
    ("pack", -2, "ATTN_ERR_ARG"), ("cus", -1, "ATTN_ERR_ARG"),
])
def test_plan_rejects(lib, field, value, want):
    kw = dict(batch=2, q_len=1, hq=8, hkv=2, d=128, page=16, maxp=512, max_L=4096)
    kw[field] = value
    code, _ = _plan(lib, **kw)
    assert L.STATUS[code] == want


def test_plan_null_arguments(lib):
    plan = L.Plan()
    assert L.STATUS[lib.attn_decode_plan(None, 0, -1, 0, ctypes.byref(plan))] == "ATTN_ERR_NULL"
    shape = L.DecodeShape(1, 1, 8, 2, 128, 16, 4, 64, 1)
    assert L.STATUS[lib.attn_decode_plan(ctypes.byref(shape), 0, -1, 0, None)] == "ATTN_ERR_NULL"


def test_dense_plan(lib):
    plan = L.Plan()
    shape = L.DenseShape(32, 32, 4, 4096, 128, 0)
    assert lib.attn_dense_plan(ctypes.byref(shape), 0, 0, ctypes.byref(plan)) == 0
    assert plan.num_splits == oplan.plan(1, 4, 32, 32, 4096, 256, 16, 128, 0, 1)[0] == 7
    shape = L.DenseShape(8, 2, 1, 512, 64, 0)
    assert lib.attn_dense_plan(ctypes.byref(shape), 0, 0, ctypes.byref(plan)) == 0
    assert plan.num_splits == 1 and plan.rows_per_unit == 4
    for bad, want in [(L.DenseShape(8, 3, 1, 512, 64, 0), "ATTN_ERR_SHAPE"),
                      (L.DenseShape(8, 2, 0, 512, 64, 0), "ATTN_ERR_SHAPE"),
                      (L.DenseShape(8, 2, 1, -1, 64, 0), "ATTN_ERR_SHAPE"),
                      (L.DenseShape(8, 2, 1, 512, 300, 0), "ATTN_ERR_UNSUPPORTED")]:
        assert L.STATUS[lib.attn_dense_plan(ctypes.byref(bad), 0, 0, ctypes.byref(plan))] == want


def test_kvcache_forward_argument_errors(lib):
    """The append / causal entry point rejects bad options before any launch."""
    P = ctypes.c_void_p
    a = P(4096)
    good = L.DecodeShape(2, 4, 8, 2, 128, 16, 8, 100, 1)
    call = lambda new_len, causal, kn=a, vn=a: L.STATUS[lib.attn_decode_kvcache_fwd(
        ctypes.byref(good), a, a, a, a, a, kn, vn, new_len, causal, 0, -1, 0.0, a, None, None, 0,
        None)]
    assert call(-1, 0) == "ATTN_ERR_ARG"
    assert call(0, 2) == "ATTN_ERR_ARG"
    assert call(3, 0, kn=None) == "ATTN_ERR_NULL"
    assert call(3, 1, vn=None) == "ATTN_ERR_NULL"
    assert call(3, 0, kn=P(4098)) == "ATTN_ERR_ALIGN"


def test_varlen_forward_argument_errors(lib):
    P = ctypes.c_void_p
    a = P(4096)
    good = L.DecodeShape(2, 4, 8, 2, 128, 16, 8, 100, 1)
    call = lambda cu, total: L.STATUS[lib.attn_decode_varlen_fwd(
        ctypes.byref(good), a, a, a, a, a, cu, total, None, None, 0, 0, 0, 0.0, a, None, None, 0,
        None)]
    assert call(None, 3) == "ATTN_ERR_NULL"
    assert call(a, 9) == "ATTN_ERR_SHAPE"   # more queries than batch * q_len
    assert call(a, -1) == "ATTN_ERR_SHAPE"
    assert call(P(4098), 3) == "ATTN_ERR_ALIGN"


def test_forward_validation_before_any_device_call(lib):
    """Argument errors return before the library touches HIP."""
    P = ctypes.c_void_p
    good = L.DecodeShape(2, 1, 8, 2, 128, 16, 4, 64, 1)
    a = P(0x10000)  # never dereferenced: every call below fails validation first
    assert L.STATUS[lib.attn_decode_fwd(None, a, a, a, a, a, 0, -1, 0.0, a, None, None, 0,
                                        None)] == "ATTN_ERR_NULL"
    assert L.STATUS[lib.attn_decode_fwd(ctypes.byref(good), None, a, a, a, a, 0, -1, 0.0, a,
                                        None, None, 0, None)] == "ATTN_ERR_NULL"
    bad = L.DecodeShape(2, 1, 8, 3, 128, 16, 4, 64, 1)
    assert L.STATUS[lib.attn_decode_fwd(ctypes.byref(bad), a, a, a, a, a, 0, -1, 0.0, a, None,
                                        None, 0, None)] == "ATTN_ERR_SHAPE"
    odd = P(0x10002)
    assert L.STATUS[lib.attn_decode_fwd(ctypes.byref(good), odd, a, a, a, a, 0, -1, 0.0, a,
                                        None, None, 0, None)] == "ATTN_ERR_ALIGN"
    assert L.STATUS[lib.attn_decode_fwd(ctypes.byref(good), a, a, a, a, a, 0, -1,
                                        float("nan"), a, None, None, 0, None)] == "ATTN_ERR_ARG"
    dshape = L.DenseShape(8, 2, 1, 512, 257, 0)
    assert L.STATUS[lib.attn_dense_fwd(ctypes.byref(dshape), a, a, a, 0, 0.0, a, None, None, 0,
                                       None)] == "ATTN_ERR_UNSUPPORTED"
    assert L.STATUS[lib.attn_combine_fwd(0, 1, 1, 8, 128, 1, a, a, a, None, None)] == \
        "ATTN_ERR_ARG"
    assert L.STATUS[lib.attn_combine_fwd(2, 1, 1, 8, 513, 1, a, a, a, None, None)] == \
        "ATTN_ERR_UNSUPPORTED"
    assert L.STATUS[lib.attn_combine_fwd(2, 1, 1, 8, 128, 1, None, a, a, None, None)] == \
        "ATTN_ERR_NULL"


def test_check_paged_inputs(lib):
    from split_kv_paged_amd import api
    bt = np.array([[0, 1, 2, 3], [4, 5, 6, 99]], dtype=np.int32)
    args = (2, 1, 8, 2, 128, 16, 4, 64, 1)
    assert api.check_paged_inputs(args, bt, np.array([64, 48], np.int32), 7) == ("ATTN_OK", -1)
    assert api.check_paged_inputs(args, bt, np.array([64, 49], np.int32), 7) == \
        ("ATTN_ERR_DATA", 1)
    assert api.check_paged_inputs(args, bt, np.array([65, 1], np.int32), 7) == \
        ("ATTN_ERR_DATA", 0)
    assert api.check_paged_inputs(args, bt, np.array([-1, 1], np.int32), 7) == \
        ("ATTN_ERR_DATA", 0)
    bt[0, 0] = -3
    assert api.check_paged_inputs(args, bt, np.array([1, 0], np.int32), 7) == \
        ("ATTN_ERR_DATA", 0)
    assert api.check_paged_inputs(args, bt, np.array([0, 0], np.int32), 7) == ("ATTN_OK", -1)
    # appended keys count against max_seqlen_k and need mapped pages
    bt[0, 0] = 0
    assert api.check_paged_inputs(args, bt, np.array([60, 40], np.int32), 7, new_len=4) == \
        ("ATTN_OK", -1)
    assert api.check_paged_inputs(args, bt, np.array([61, 40], np.int32), 7, new_len=4) == \
        ("ATTN_ERR_DATA", 0)
    assert api.check_paged_inputs(args, bt, np.array([60, 45], np.int32), 7, new_len=4) == \
        ("ATTN_ERR_DATA", 1)
    assert api.check_paged_inputs(args, bt, np.array([0, 0], np.int32), 7, new_len=-1) == \
        ("ATTN_ERR_ARG", -1)
    # the plain check is the same with new_len = 0, through its own symbol
    shape = L.DecodeShape(*args)
    sl = np.array([64, 48], np.int32)
    bad = ctypes.c_int32(-1)
    assert lib.attn_check_paged_inputs(ctypes.byref(shape), bt.ctypes.data_as(ctypes.c_void_p),
                                       sl.ctypes.data_as(ctypes.c_void_p), 7,
                                       ctypes.byref(bad)) == 0


# The ragged-batch refinement (not from the pages): with the sum of the
# lengths given, the planner takes max(page rule, ceil(max_L / (share / 2)))
# when max_L > 2 * mean and max_L > 2 * share, share = streams * sum_L / CUs,
# streams = head units x row blocks.  Expected values worked by hand for the
# shapes below.
RAGGED_CASES = [
    # (name, kwargs, expected S)
    # 128 seqs, 16 q heads / 8 KV heads, d 64 as 4 head pairs: share =
    # 4 * 112861 / 256 = 1763.45; 7769 > 1.5 * 1763.45 = 2645.2;
    # ceil(5 * 7769 / (3 * 1763.45)) = ceil(7.34) = 8; page rule alone: 1
    ("ragged d64", dict(batch=128, q_len=1, hq=16, hkv=8, d=64, maxp=512, max_L=7769,
                        sum_L=112861), 8),
    # 32 seqs GQA-4 d 128: share = 8 * 40957 / 256 = 1279.9;
    # ceil(5 * 6642 / (3 * 1279.9)) = ceil(8.65) = 9
    ("ragged d128", dict(batch=32, q_len=1, hq=32, hkv=8, maxp=416, max_L=6642, sum_L=40957), 9),
    # near-uniform lengths: share = 8 * 32002 / 256 = 1000.06; 1100 <= 2000: rule's 1
    ("uniform ~1000", dict(batch=32, q_len=1, hq=32, hkv=8, maxp=69, max_L=1100, sum_L=32002), 1),
    # long uniform context, GQA-8: max_L = mean, not ragged: the rule's 14
    # leaves 256 - 16 * 14 = 32 CUs idle; with the sum, 256 / 16 = 16
    ("long uniform", dict(batch=4, q_len=1, hq=32, hkv=4, maxp=1024, max_L=16384, sum_L=65536), 16),
    # ragged but short against the share: mean 1000, max 2400 > 2000, share
    # 8 * 64000 / 256 = 2000, 2400 <= 1.5 * 2000: the rule's 1
    ("ragged under 1.5 shares", dict(batch=64, q_len=1, hq=32, hkv=8, maxp=150, max_L=2400,
                                     sum_L=64000), 1),
    # one long sequence among 255 one-key ones: share = 65791 / 256 = 257.0,
    # ceil(5 * 65536 / (3 * 257.0)) = 426 pieces asked, capped at 128
    ("cap", dict(batch=256, q_len=1, hq=1, hkv=1, maxp=4096, max_L=65536, sum_L=65536 + 255), 128),
    # 32 query rows per unit (q_len 8, G 4): two row blocks of 16 would be one
    # 32-row block, streams = 8: share = 8 * 40957 / 256, as in "ragged d128"
    ("ragged 32 rows", dict(batch=32, q_len=8, hq=32, hkv=8, maxp=416, max_L=6642,
                            sum_L=40957), 9),
]


@pytest.mark.parametrize("name,kw,want", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_ragged_hint_plan(lib, name, kw, want):
    code, plan = _plan(lib, **kw)
    assert L.STATUS[code] == "ATTN_OK"
    assert plan.num_splits == want, (name, plan.num_splits)
    # without the hint the pages' rule alone decides
    kw0 = dict(kw, sum_L=0)
    code0, plan0 = _plan(lib, **kw0)
    hkv = kw["hkv"] // plan0.heads_per_row  # the rule counts head groups
    ref_splits, _ = oplan.plan(kw["batch"], kw["q_len"], kw["hq"], hkv, kw["max_L"], 256, 16,
                               128, unit_block_m=unit_tile(kw["q_len"], kw["hq"] // hkv, -1))
    assert plan0.num_splits == ref_splits
    assert plan.num_splits >= plan0.num_splits


# Compact list: extra_blocks = max(1, floor(sum / C) * head units * row
# blocks), used when units + extra_blocks < units * S.  Worked by hand:
#   ragged d64:  4 head pairs; C = 16 * ceil(486 / 8) = 976;
#                floor(112861 / 976) = 115; 115 * 4 = 460; 512 + 460 = 972 < 4096
#   ragged d128: C = 16 * ceil(416 / 9) = 752; floor(40957 / 752) = 54;
#                54 * 8 = 432; 256 + 432 = 688 < 2304
#   long uniform: C = 1024; floor(65536 / 1024) * 4 = 256; 16 + 256 = 272 is
#                not below 16 * 16 = 256: split-major
#   cap:         C = 512; floor(65791 / 512) = 128; 256 + 128 < 32768
#   ragged 32 rows: as ragged d128 (one 32-row block per unit)
COMPACT_EXTRA = {"ragged d64": 460, "ragged d128": 432, "uniform ~1000": 0, "long uniform": 0,
                 "ragged under 1.5 shares": 0, "cap": 128, "ragged 32 rows": 432}


@pytest.mark.parametrize("name,kw,want", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_compact_list_plan(lib, name, kw, want):
    code, plan = _plan(lib, **kw)
    assert L.STATUS[code] == "ATTN_OK"
    assert plan.extra_blocks == COMPACT_EXTRA[name]
    if plan.extra_blocks:
        assert plan.grid == plan.units + plan.extra_blocks < plan.units * plan.num_splits
    else:
        assert plan.grid == plan.units * plan.num_splits
    # the compact list changes the grid only: same splits and partials (head
    # pairs, which also wait for the sum, halve the arrival counters)
    code0, plan0 = _plan(lib, **dict(kw, sum_L=0, S=plan.num_splits))
    assert plan0.extra_blocks == 0 and plan0.grid == plan0.units * plan0.num_splits
    counters = lambda p: (p.units * 128 + 255) // 256 * 256 if p.num_splits > 1 else 0
    assert (plan0.workspace_bytes - counters(plan0)) == (plan.workspace_bytes - counters(plan))
    assert plan0.units == plan.units * plan.heads_per_row
    assert plan0.split_keys == plan.split_keys
    # a batch over 1024 sequences keeps the split-major grid
    if plan.num_splits > 1:
        big = dict(kw, batch=1100, sum_L=kw["sum_L"] * 1100 // kw["batch"], S=plan.num_splits)
        code2, plan2 = _plan(lib, **big)
        assert L.STATUS[code2] == "ATTN_OK" and plan2.extra_blocks == 0


FILL_CASES = [
    # (name, kwargs, S with the sum, S of the pages' rule)
    # 16 units (4 x 4 KV heads): 14 * 16 = 224 < 256 CUs; 256 / 16 = 16
    ("long context", dict(batch=4, q_len=1, hq=32, hkv=4, maxp=1024, max_L=16384), 16, 14),
    # 16 units again, 4000 keys: 4000 / 128 = 31 keys-wise, so 16
    ("two sequences", dict(batch=2, q_len=1, hq=32, hkv=8, maxp=250, max_L=4000), 16, 14),
    # 8 units, 1000 keys: 256 / 8 = 32, but 1000 / 128 = 7 tiles of 8 waves: stays 7
    ("short", dict(batch=1, q_len=1, hq=32, hkv=8, maxp=63, max_L=1000), 7, 7),
    # 4 units, 65536 keys: 64 asked by the CUs, capped at 16 (one round of loads)
    ("cap 16", dict(batch=1, q_len=1, hq=32, hkv=4, maxp=4096, max_L=65536), 16, None),
]


@pytest.mark.parametrize("name,kw,want,rule", FILL_CASES, ids=[c[0] for c in FILL_CASES])
def test_fill_the_cus_with_the_sum(lib, name, kw, want, rule):
    """With the length sum (uniform lengths here), a split count that leaves
    CUs idle is raised to fill them, up to 16 splits and down to 128 keys a
    split; without it the plan is the pages' rule."""
    code, plan = _plan(lib, **dict(kw, sum_L=kw["batch"] * kw["max_L"]))
    assert L.STATUS[code] == "ATTN_OK"
    code0, plan0 = _plan(lib, **kw)
    assert L.STATUS[code0] == "ATTN_OK"
    if rule is not None:
        assert plan0.num_splits == rule
    assert plan.num_splits == max(want, plan0.num_splits)


def test_ragged_hint_rejects_out_of_range(lib):
    base = dict(batch=4, q_len=1, hq=8, hkv=2, maxp=64, max_L=1000)
    assert L.STATUS[_plan(lib, **base, sum_L=-1)[0]] == "ATTN_ERR_SHAPE"
    assert L.STATUS[_plan(lib, **base, sum_L=4001)[0]] == "ATTN_ERR_SHAPE"
    assert L.STATUS[_plan(lib, **base, sum_L=4000)[0]] == "ATTN_OK"
    # an explicit split count is never changed by the hint
    code, plan = _plan(lib, batch=128, q_len=1, hq=16, hkv=8, d=64, maxp=512, max_L=7769,
                       sum_L=112861, S=3)
    assert L.STATUS[code] == "ATTN_OK" and plan.num_splits == 3
