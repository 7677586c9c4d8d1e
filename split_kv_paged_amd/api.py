"""torch-facing binding of the C ABI.

PyTorch provides device memory and the stream; every step of the attention
runs in the library's HIP kernels.  Functions here check tensor placement,
dtype and layout, allocate outputs / workspace with torch when the caller
does not pass them, and call the library on torch's current stream, or on
the stream the caller passes: then the outputs and the zero-filled workspace
are allocated and filled on that stream too, so the fill is ordered before
the kernel that relies on it.
"""
import contextlib
import ctypes

import torch

from . import lib as _L

_DT = {torch.float16: _L.FP16, torch.bfloat16: _L.BF16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context: the caller's stream when one is given."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def decode_shape(q, k_cache, block_table, max_seqlen_k=None, sum_seqlen_k=None):
    B, qlen, hq, d = q.shape
    _, page, hkv, d2 = k_cache.shape
    _need(d2 == d, "q and k_cache head_dim differ")
    maxp = block_table.shape[1]
    if max_seqlen_k is None:
        max_seqlen_k = maxp * page
    return _L.DecodeShape(B, qlen, hq, hkv, d, page, maxp, int(max_seqlen_k), _DT[q.dtype],
                          int(sum_seqlen_k or 0))


def decode_plan(batch, q_len, num_heads_q, num_heads_kv, head_dim, page_size, max_pages_per_seq,
                max_seqlen_k, dtype=torch.bfloat16, num_splits=0, pack_gqa=-1, num_cus=0,
                sum_seqlen_k=0):
    """Host-only plan (no device touched)."""
    shape = _L.DecodeShape(batch, q_len, num_heads_q, num_heads_kv, head_dim, page_size,
                           max_pages_per_seq, max_seqlen_k,
                           _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
                           int(sum_seqlen_k))
    plan = _L.Plan()
    _L.check("attn_decode_plan",
             _L.load().attn_decode_plan(ctypes.byref(shape), num_splits, pack_gqa, num_cus,
                                        ctypes.byref(plan)))
    return plan


def dense_plan(num_heads_q, num_heads_kv, q_len, kv_len, head_dim, dtype=torch.float16,
               num_splits=0, num_cus=0):
    shape = _L.DenseShape(num_heads_q, num_heads_kv, q_len, kv_len, head_dim,
                          _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype))
    plan = _L.Plan()
    _L.check("attn_dense_plan",
             _L.load().attn_dense_plan(ctypes.byref(shape), num_splits, num_cus,
                                       ctypes.byref(plan)))
    return plan


def last_plan():
    plan = _L.Plan()
    _L.check("attn_last_plan", _L.load().attn_last_plan(ctypes.byref(plan)))
    return plan


def _check_dev(*ts):
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        _need(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
        _need(t.is_contiguous(), "tensors must be contiguous")
    return dev


def decode_fwd(q, k_cache, v_cache, block_table, cache_seqlens, num_splits=0, pack_gqa=-1,
               softmax_scale=None, max_seqlen_k=None, out=None, lse=None, return_lse=True,
               workspace=None, stream=None, k_new=None, v_new=None, causal=False,
               sum_seqlen_k=None):
    """Paged decode attention.

    q [B, q_len, Hq, d] fp16/bf16; k_cache, v_cache [pages, page, Hkv, d];
    block_table int32 [B, max_pages]; cache_seqlens int32 [B].
    Returns (out [B, q_len, Hq, d], lse float32 [B, Hq, q_len] or None).
    max_seqlen_k (a host int bound on the attended lengths) drives the plan;
    by default it is max_pages * page_size, which needs no device sync.  A
    tight bound matters for speed: the split count, the split length and
    the longest-first ordering are all chosen from it.
    k_new / v_new [B, new_len, Hkv, d]: keys written into the cache at
    positions cache_seqlens[b].. before attention (attn_decode_kvcache_fwd);
    causal: query i of q_len sees keys j <= L - q_len + i.
    sum_seqlen_k (optional host int, the sum of the attended lengths) lets
    an automatic plan split the longest sequences of a ragged batch.
    """
    _need(q.dtype in _DT and k_cache.dtype == q.dtype and v_cache.dtype == q.dtype,
          "q, k_cache, v_cache must share fp16 or bf16")
    _need(block_table.dtype == torch.int32 and cache_seqlens.dtype == torch.int32,
          "block_table and cache_seqlens must be int32")
    dev = _check_dev(q, k_cache, v_cache, block_table, cache_seqlens, out, lse, workspace)
    shape = decode_shape(q, k_cache, block_table, max_seqlen_k, sum_seqlen_k)
    lib = _L.load()
    plan = _L.Plan()
    with torch.cuda.device(dev), _on(stream):
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        _L.check("attn_decode_plan", lib.attn_decode_plan(ctypes.byref(shape), num_splits,
                                                          pack_gqa, cus, ctypes.byref(plan)))
        if out is None:
            out = torch.empty_like(q)
        if lse is None and return_lse:
            lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                              device=dev)
        if workspace is None and plan.workspace_bytes > 0:
            # zero-filled: the fused combine's arrival counters start at zero
            workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        if k_new is None and not causal:
            name = "attn_decode_fwd"
            code = lib.attn_decode_fwd(
                ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                _ptr(cache_seqlens), num_splits, pack_gqa,
                float(softmax_scale) if softmax_scale else 0.0, _ptr(out), _ptr(lse),
                _ptr(workspace), ws_bytes, _stream(dev, stream))
        else:
            name = "attn_decode_kvcache_fwd"
            new_len = 0
            if k_new is not None:
                _need(v_new is not None and k_new.shape == v_new.shape and k_new.dim() == 4
                      and k_new.shape[0] == q.shape[0] and k_new.shape[2:] == k_cache.shape[2:]
                      and k_new.dtype == q.dtype and v_new.dtype == q.dtype
                      and k_new.is_contiguous() and v_new.is_contiguous()
                      and k_new.device == dev and v_new.device == dev,
                      "k_new / v_new must be contiguous [B, new_len, Hkv, d] of q's dtype")
                new_len = int(k_new.shape[1])
            code = lib.attn_decode_kvcache_fwd(
                ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                _ptr(cache_seqlens), _ptr(k_new), _ptr(v_new), new_len, int(bool(causal)),
                num_splits, pack_gqa, float(softmax_scale) if softmax_scale else 0.0, _ptr(out),
                _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev, stream))
    _L.check(name, code)
    return out, lse


def decode_varlen_fwd(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q,
                      max_seqlen_q, num_splits=0, softmax_scale=None, max_seqlen_k=None,
                      out=None, lse=None, return_lse=True, workspace=None, stream=None,
                      k_new=None, v_new=None, causal=False, sum_seqlen_k=None):
    """Paged decode attention with a query count per sequence.

    q [total_q, Hq, d]; cu_seqlens_q int32 [B + 1] on the device (queries of
    sequence b are rows cu[b]..cu[b+1]-1, at most max_seqlen_q of them).
    Returns (out [total_q, Hq, d], lse float32 [Hq, total_q] or None).
    """
    _need(q.dim() == 3 and q.dtype in _DT and k_cache.dtype == q.dtype
          and v_cache.dtype == q.dtype, "q [total_q, Hq, d]; q, k_cache, v_cache share a dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.numel() == block_table.shape[0] + 1,
          "cu_seqlens_q must be int32 [B + 1]")
    dev = _check_dev(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, out, lse,
                     workspace)
    total_q, hq, d = q.shape
    B = block_table.shape[0]
    pages, page, hkv, d2 = k_cache.shape
    _need(d2 == d, "head_dim")
    maxp = block_table.shape[1]
    shape = _L.DecodeShape(B, int(max_seqlen_q), hq, hkv, d, page, maxp,
                           int(max_seqlen_k if max_seqlen_k is not None else maxp * page),
                           _DT[q.dtype], int(sum_seqlen_k or 0))
    lib = _L.load()
    plan = _L.Plan()
    new_len = 0
    if k_new is not None:
        _need(v_new is not None and k_new.shape == v_new.shape and k_new.dim() == 4
              and k_new.shape[0] == B and k_new.shape[2:] == k_cache.shape[2:]
              and k_new.dtype == q.dtype and v_new.dtype == q.dtype and k_new.is_contiguous()
              and v_new.is_contiguous(), "k_new / v_new must be contiguous [B, new_len, Hkv, d]")
        new_len = int(k_new.shape[1])
    with torch.cuda.device(dev), _on(stream):
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        _L.check("attn_decode_plan", lib.attn_decode_plan(ctypes.byref(shape), num_splits, 1,
                                                          cus, ctypes.byref(plan)))
        if out is None:
            out = torch.empty_like(q)
        if lse is None and return_lse:
            lse = torch.empty((hq, total_q), dtype=torch.float32, device=dev)
        if workspace is None and plan.workspace_bytes > 0:
            workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        code = lib.attn_decode_varlen_fwd(
            ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(cache_seqlens), _ptr(cu_seqlens_q), int(total_q), _ptr(k_new), _ptr(v_new),
            new_len, int(bool(causal)), num_splits,
            float(softmax_scale) if softmax_scale else 0.0, _ptr(out), _ptr(lse),
            _ptr(workspace), ws_bytes, _stream(dev, stream))
    _L.check("attn_decode_varlen_fwd", code)
    return out, lse


def dense_fwd(q, k, v, num_splits=0, softmax_scale=None, out=None, lse=None, return_lse=True,
              workspace=None, stream=None):
    """Dense small-query attention: q [Hq, q_len, d], k/v [Hkv, kv_len, d].

    Returns (out [Hq, q_len, d], lse float32 [Hq, q_len] or None).
    """
    _need(q.dtype in _DT and k.dtype == q.dtype and v.dtype == q.dtype,
          "q, k, v must share fp16 or bf16")
    dev = _check_dev(q, k, v, out, lse, workspace)
    hq, qlen, d = q.shape
    hkv, kvlen, d2 = k.shape
    _need(d2 == d and tuple(v.shape) == tuple(k.shape), "k/v shapes")
    shape = _L.DenseShape(hq, hkv, qlen, kvlen, d, _DT[q.dtype])
    lib = _L.load()
    plan = _L.Plan()
    with torch.cuda.device(dev), _on(stream):
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        _L.check("attn_dense_plan", lib.attn_dense_plan(ctypes.byref(shape), num_splits, cus,
                                                        ctypes.byref(plan)))
        if out is None:
            out = torch.empty_like(q)
        if lse is None and return_lse:
            lse = torch.empty((hq, qlen), dtype=torch.float32, device=dev)
        if workspace is None and plan.workspace_bytes > 0:
            workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        code = lib.attn_dense_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), num_splits,
                                  float(softmax_scale) if softmax_scale else 0.0, _ptr(out),
                                  _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev, stream))
    _L.check("attn_dense_fwd", code)
    return out, lse


def combine_fwd(o_part, lse_part, batch, q_len, num_heads, dtype=torch.bfloat16, out=None,
                lse=None, stream=None):
    """Merge partials: o_part float32 [S, rows, d], lse_part float32 [S, rows],
    rows ordered (b, i, h).  Returns (out [batch, q_len, heads, d], lse [batch, heads, q_len])."""
    _need(o_part.dtype == torch.float32 and lse_part.dtype == torch.float32, "float32 partials")
    S, rows, d = o_part.shape
    _need(rows == batch * q_len * num_heads and tuple(lse_part.shape) == (S, rows), "shapes")
    dev = _check_dev(o_part, lse_part, out, lse)
    with torch.cuda.device(dev), _on(stream):
        if out is None:
            out = torch.empty((batch, q_len, num_heads, d), dtype=dtype, device=dev)
        if lse is None:
            lse = torch.empty((batch, num_heads, q_len), dtype=torch.float32, device=dev)
        code = _L.load().attn_combine_fwd(S, batch, q_len, num_heads, d, _DT[out.dtype],
                                          _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse),
                                          _stream(dev, stream))
    _L.check("attn_combine_fwd", code)
    return out, lse


def workspace_partials(workspace, plan, nrows, head_dim):
    """Views of the float32 partials a split call left in its workspace:
    (o_part [S, nrows, d], lse_part [S, nrows])."""
    S = plan.num_splits
    o_bytes = (S * nrows * head_dim * 4 + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    o = f[:S * nrows * head_dim * 4].view(torch.float32).view(S, nrows, head_dim)
    l = f[o_bytes:o_bytes + S * nrows * 4].view(torch.float32).view(S, nrows)
    return o, l


def check_paged_inputs(shape_args, block_table_host, cache_seqlens_host, num_pages, new_len=0):
    """Host check of block_table / cache_seqlens ranges (numpy int32 arrays),
    for a call that appends new_len keys per sequence (0: a plain decode
    call).  Returns (status_name, bad_batch)."""
    import numpy as np
    shape = _L.DecodeShape(*shape_args)
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    sl = np.ascontiguousarray(cache_seqlens_host, dtype=np.int32)
    bad = ctypes.c_int32(-1)
    code = _L.load().attn_check_kvcache_inputs(ctypes.byref(shape),
                                               bt.ctypes.data_as(ctypes.c_void_p),
                                               sl.ctypes.data_as(ctypes.c_void_p),
                                               int(num_pages), int(new_len), ctypes.byref(bad))
    return _L.STATUS[code], bad.value


class PreparedDecode:
    """A decode call with its arguments marshalled once, for tight loops.

    Holds the shape struct and pointers of one set of tensors; each call
    re-enters attn_decode_fwd (which plans and validates again on the host)
    with only the KV pointers optionally swapped; with causal or k_new /
    v_new (keys appended at cache_seqlens[b].., as in decode_fwd) it is
    attn_decode_kvcache_fwd.  The tensors must stay alive and keep their
    shapes for the object's lifetime.
    """

    def __init__(self, q, k_cache, v_cache, block_table, cache_seqlens, num_splits=0,
                 pack_gqa=-1, softmax_scale=None, max_seqlen_k=None, out=None, lse=None,
                 workspace=None, stream=None, causal=False, sum_seqlen_k=None, k_new=None,
                 v_new=None):
        _need(q.dtype in _DT and k_cache.dtype == q.dtype and v_cache.dtype == q.dtype,
              "q, k_cache, v_cache must share fp16 or bf16")
        dev = _check_dev(q, k_cache, v_cache, block_table, cache_seqlens, out, lse, workspace)
        new_len = 0
        if k_new is not None:
            _need(v_new is not None and k_new.shape == v_new.shape and k_new.dim() == 4
                  and k_new.shape[0] == q.shape[0] and k_new.shape[2:] == k_cache.shape[2:]
                  and k_new.dtype == q.dtype and v_new.dtype == q.dtype
                  and k_new.is_contiguous() and v_new.is_contiguous()
                  and k_new.device == dev and v_new.device == dev,
                  "k_new / v_new must be contiguous [B, new_len, Hkv, d] of q's dtype")
            new_len = int(k_new.shape[1])
        self.shape = decode_shape(q, k_cache, block_table, max_seqlen_k, sum_seqlen_k)
        self.lib = _L.load()
        plan = _L.Plan()
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        _L.check("attn_decode_plan", self.lib.attn_decode_plan(
            ctypes.byref(self.shape), num_splits, pack_gqa, cus, ctypes.byref(plan)))
        self.plan = plan
        with torch.cuda.device(dev), _on(stream):
            self.out = out if out is not None else torch.empty_like(q)
            self.lse = lse if lse is not None else torch.empty(
                (q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=dev)
            if workspace is None and plan.workspace_bytes > 0:
                workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self._keep = (q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new)
        tail = [int(num_splits), int(pack_gqa), float(softmax_scale) if softmax_scale else 0.0,
                _ptr(self.out), _ptr(self.lse), _ptr(workspace),
                workspace.numel() if workspace is not None else 0, _stream(dev, stream)]
        head = [ctypes.byref(self.shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                _ptr(block_table), _ptr(cache_seqlens)]
        if causal or new_len:  # attn_decode_kvcache_fwd
            self.args = head + [_ptr(k_new), _ptr(v_new), new_len, int(bool(causal))] + tail
            self.fn = self.lib.attn_decode_kvcache_fwd
        else:
            self.args = head + tail
            self.fn = self.lib.attn_decode_fwd

    def __call__(self, k_cache=None, v_cache=None):
        a = self.args
        if k_cache is not None:
            a = list(a)
            a[2] = ctypes.c_void_p(k_cache.data_ptr())
            a[3] = ctypes.c_void_p(v_cache.data_ptr())
        code = self.fn(*a)
        if code:
            _L.check(self.fn.__name__, code)
        return self.out, self.lse


class PreparedDense:
    """A dense call with its arguments marshalled once, for tight loops (see
    PreparedDecode); each call re-enters attn_dense_fwd with optionally
    swapped K/V pointers."""

    def __init__(self, q, k, v, num_splits=0, softmax_scale=None, out=None, lse=None,
                 workspace=None, stream=None):
        _need(q.dtype in _DT and k.dtype == q.dtype and v.dtype == q.dtype,
              "q, k, v must share fp16 or bf16")
        dev = _check_dev(q, k, v, out, lse, workspace)
        hq, qlen, d = q.shape
        hkv, kvlen, d2 = k.shape
        _need(d2 == d and tuple(v.shape) == tuple(k.shape), "k/v shapes")
        self.shape = _L.DenseShape(hq, hkv, qlen, kvlen, d, _DT[q.dtype])
        self.lib = _L.load()
        plan = _L.Plan()
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        _L.check("attn_dense_plan", self.lib.attn_dense_plan(
            ctypes.byref(self.shape), num_splits, cus, ctypes.byref(plan)))
        self.plan = plan
        with torch.cuda.device(dev), _on(stream):
            self.out = out if out is not None else torch.empty_like(q)
            self.lse = lse if lse is not None else torch.empty((hq, qlen), dtype=torch.float32,
                                                               device=dev)
            if workspace is None and plan.workspace_bytes > 0:
                workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self._keep = (q, k, v)
        self.args = [ctypes.byref(self.shape), _ptr(q), _ptr(k), _ptr(v), int(num_splits),
                     float(softmax_scale) if softmax_scale else 0.0, _ptr(self.out),
                     _ptr(self.lse), _ptr(workspace),
                     workspace.numel() if workspace is not None else 0, _stream(dev, stream)]
        self.fn = self.lib.attn_dense_fwd

    def __call__(self, k=None, v=None):
        a = self.args
        if k is not None:
            a = list(a)
            a[2] = ctypes.c_void_p(k.data_ptr())
            a[3] = ctypes.c_void_p(v.data_ptr())
        code = self.fn(*a)
        if code:
            _L.check("attn_dense_fwd", code)
        return self.out, self.lse
