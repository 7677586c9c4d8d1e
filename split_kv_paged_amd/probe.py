"""ctypes binding of the read-only bandwidth probes (include/attn_probe.h).

Measurement helpers: they read the same KV bytes as a decode call and fold
them into 32-bit word sums, nothing else, so their speed is the ceiling a
decode call is compared with.  Loading fails loudly when libattn_probe.so
has not been built.
"""
import ctypes
import os

import torch

from . import lib as _L

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_probe.so")
EXPORTS = ("attn_probe_stream_read", "attn_probe_page_read")

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libattn_probe.so is not built (expected at %s); run "
                           "`python -m split_kv_paged_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.attn_probe_stream_read.argtypes = [P, Z, P, Z, P, I, P]
    lib.attn_probe_stream_read.restype = I
    lib.attn_probe_page_read.argtypes = [ctypes.POINTER(_L.DecodeShape), P, P, P, P, I, P, P]
    lib.attn_probe_page_read.restype = I
    _lib = lib
    return lib


def _check(fn, code):
    if code != _L.ATTN_OK:
        raise _L.AttnError(fn, code, _L.STATUS.get(code, str(code)))


def _stream(dev, stream):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def prepared_stream_read(a, b, a_bytes=None, b_bytes=None, num_blocks=512, sums=None,
                         stream=None):
    """Check the arguments once and return (call, sums): call() enqueues a
    read of the first a_bytes of tensor a and b_bytes of tensor b (default:
    all of each, rounded down to 16 bytes); sums is the int32 tensor of
    per-workgroup word sums (their sum mod 2^32 is the checksum)."""
    a_bytes = a.numel() * a.element_size() if a_bytes is None else int(a_bytes)
    b_bytes = b.numel() * b.element_size() if b_bytes is None else int(b_bytes)
    a_bytes -= a_bytes % 16
    b_bytes -= b_bytes % 16
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("stream_read needs contiguous tensors")
    if a_bytes > a.numel() * a.element_size() or b_bytes > b.numel() * b.element_size():
        raise ValueError("stream_read range exceeds the tensor")
    if sums is None:
        sums = torch.empty(num_blocks, dtype=torch.int32, device=a.device)
    if sums.numel() < num_blocks or sums.dtype != torch.int32 or not sums.is_contiguous():
        raise ValueError("sums must be a contiguous int32 tensor of %d elements" % num_blocks)
    fn = load().attn_probe_stream_read
    args = (ctypes.c_void_p(a.data_ptr()), a_bytes, ctypes.c_void_p(b.data_ptr()), b_bytes,
            ctypes.c_void_p(sums.data_ptr()), num_blocks, _stream(a.device, stream))

    def call():
        _check("attn_probe_stream_read", fn(*args))
    return call, sums


def stream_read(a, b, a_bytes=None, b_bytes=None, num_blocks=512, sums=None, stream=None):
    """One stream read (see prepared_stream_read); returns the sums tensor."""
    call, sums = prepared_stream_read(a, b, a_bytes, b_bytes, num_blocks, sums, stream)
    call()
    return sums


def prepared_page_read(k_cache, v_cache, block_table, cache_seqlens, max_seqlen_k=None,
                       split_keys=0, sums=None, stream=None):
    """Check the arguments once and return (call, sums): call() enqueues a
    read of the valid keys' K and V rows the way the decode kernel walks the
    pages, split into ranges of split_keys keys (0: one range); sums is int32
    [S, batch, num_heads_kv] of word sums."""
    for t in (k_cache, v_cache, block_table, cache_seqlens):
        if not t.is_contiguous():
            raise ValueError("page_read needs contiguous tensors")
    if k_cache.shape != v_cache.shape or k_cache.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("k_cache / v_cache must match and be fp16 or bf16")
    if block_table.dtype != torch.int32 or cache_seqlens.dtype != torch.int32:
        raise ValueError("block_table and cache_seqlens must be int32")
    _, page, hkv, d = k_cache.shape
    B, maxp = block_table.shape
    if max_seqlen_k is None:
        max_seqlen_k = maxp * page
    split_keys = int(split_keys)
    S = -(-int(max_seqlen_k) // split_keys) if split_keys > 0 and max_seqlen_k > 0 else 1
    shape = _L.DecodeShape(B, 1, hkv, hkv, d, page, maxp, int(max_seqlen_k),
                           _L.BF16 if k_cache.dtype == torch.bfloat16 else _L.FP16, 0)
    if sums is None:
        sums = torch.empty(S, B, hkv, dtype=torch.int32, device=k_cache.device)
    if sums.numel() < S * B * hkv or sums.dtype != torch.int32 or not sums.is_contiguous():
        raise ValueError("sums must be a contiguous int32 tensor of %d elements" % (S * B * hkv))
    fn = load().attn_probe_page_read
    args = (ctypes.byref(shape), ctypes.c_void_p(k_cache.data_ptr()),
            ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(block_table.data_ptr()),
            ctypes.c_void_p(cache_seqlens.data_ptr()), split_keys,
            ctypes.c_void_p(sums.data_ptr()), _stream(k_cache.device, stream))

    def call():
        _check("attn_probe_page_read", fn(*args))
    call.shape = shape  # keeps the struct that args point to alive
    return call, sums


def page_read(k_cache, v_cache, block_table, cache_seqlens, max_seqlen_k=None, split_keys=0,
              sums=None, stream=None):
    """One page read (see prepared_page_read); returns the sums tensor."""
    call, sums = prepared_page_read(k_cache, v_cache, block_table, cache_seqlens, max_seqlen_k,
                                    split_keys, sums, stream)
    call()
    return sums
