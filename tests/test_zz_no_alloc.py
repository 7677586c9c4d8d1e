"""GPU: attn_decode_fwd_noalloc (library-held scratch) against attn_decode_fwd.

Both entry points run the same kernels; the no-allocation one keeps a split
call's partials and arrival counters in the library's per-GPU scratch array
instead of the caller's workspace.  Two split calls in a row (the second
smaller, with another split count, so the partials land at other offsets)
must equal attn_decode_fwd bit for bit and the float64 oracle within the
output tolerances; an unsplit call too; a call whose partials exceed the
scratch is refused before anything is launched.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from split_kv_paged_amd import api
from split_kv_paged_amd import lib as L
from split_kv_paged_amd import workloads as W
from tests.parity import bits_of, check_lse, check_out, i32_dev, to_dev

pytestmark = pytest.mark.gpu


def case(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(wl, q, kc, vc, bt, sl, num_splits):
    """One attn_decode_fwd_noalloc call through the C ABI, outputs allocated here."""
    shape = api.decode_shape(q, kc, bt, wl.max_seqlen_k, None)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), dtype=torch.float32,
                     device=q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = L.load().attn_decode_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(kc), _ptr(vc),
                                            _ptr(bt), _ptr(sl), num_splits, -1,
                                            ctypes.c_float(wl.scale), _ptr(out), _ptr(lse),
                                            stream)
    L.check("attn_decode_fwd_noalloc", code)
    torch.cuda.synchronize()
    return bits_of(out), lse.cpu().numpy(), api.last_plan()


def _both(wl, num_splits):
    q, kc, vc = (to_dev(a, wl.dtype) for a in (wl.q, wl.k_cache, wl.v_cache))
    bt, sl = i32_dev(wl.block_table), i32_dev(wl.cache_seqlens)
    o1, l1, p1 = _noalloc(wl, q, kc, vc, bt, sl, num_splits)
    out, lse = api.decode_fwd(q, kc, vc, bt, sl, num_splits=num_splits, softmax_scale=wl.scale,
                              max_seqlen_k=wl.max_seqlen_k)
    torch.cuda.synchronize()
    o2, l2, p2 = bits_of(out), lse.cpu().numpy(), api.last_plan()
    assert p1.num_splits == p2.num_splits and p1.grid == p2.grid
    return (o1, l1, p1), (o2, l2)


def _check(wl, num_splits, want_split):
    (o1, l1, plan), (o2, l2) = _both(wl, num_splits)
    assert (plan.num_splits > 1) == want_split, plan.num_splits
    assert np.array_equal(o1, o2), "noalloc output differs from attn_decode_fwd"
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), "noalloc LSE differs"
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, wl.dtype, scale=wl.scale)
    e1 = check_out(o1, ref_o, wl.dtype, "noalloc S=%d" % plan.num_splits)
    e2 = check_lse(l1, ref_l)
    print("  S=%d grid=%d max|dO|=%.3g max|dLSE|=%.3g" % (plan.num_splits, plan.grid, e1, e2),
          flush=True)


def test_noalloc_two_calls_match_workspace_path():
    case("noalloc: bf16 B4 Hq32/Hkv4 d128 L 3000..4096, planner splits, then a smaller "
         "fp16 B2 Hq16/Hkv2 d64 call at S=3, then an unsplit call")
    big = W.make_paged(7101, "bf16", 4, 1, 32, 4, 128, 16, [4096, 3001, 3500, 4000],
                       name="noalloc-big")
    _check(big, 0, True)
    small = W.make_paged(7102, "fp16", 2, 1, 16, 2, 64, 16, [700, 1000], name="noalloc-small")
    _check(small, 3, True)
    one = W.make_paged(7103, "bf16", 3, 1, 16, 4, 128, 16, [1, 130, 517], name="noalloc-one")
    _check(one, 1, False)
    # the big call again after the smaller ones: counters left at zero, partials overwritten
    _check(big, 0, True)


def test_noalloc_refuses_calls_beyond_the_scratch():
    case("noalloc: a split call whose partials exceed the scratch is refused")
    # 128 sequences x 32 query heads x head_dim 128 = 2 MiB of partials per split
    shape = L.DecodeShape(128, 1, 32, 8, 128, 16, 64, 1024, L.BF16, 0)
    plan = L.Plan()
    L.check("attn_decode_plan",
            L.load().attn_decode_plan(ctypes.byref(shape), 8, -1, 0, ctypes.byref(plan)))
    assert plan.num_splits == 8
    dev = torch.device("cuda:0")
    q = torch.zeros((128, 1, 32, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((16, 16, 8, 128), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((128, 64), dtype=torch.int32, device=dev)
    sl = torch.zeros(128, dtype=torch.int32, device=dev)
    out = torch.zeros_like(q)
    code = L.load().attn_decode_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(kc), _ptr(kc),
                                            _ptr(bt), _ptr(sl), 8, -1, ctypes.c_float(0.0),
                                            _ptr(out), None, None)
    assert L.STATUS[code] == "ATTN_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
