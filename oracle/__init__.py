"""float64 CPU oracle for exact decode / small-query attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the library itself never does.
It shares no code with the GPU library: the arithmetic lives in
``attn_oracle.c`` (plain C, float64) and in ``planner.py`` (the pages'
pack_gqa / num_splits rules, plain Python).

Every function here takes host numpy arrays.  16-bit inputs are passed as
their raw bit patterns (``uint16``) together with a dtype tag, so the oracle
sees exactly the bytes the GPU sees.

Parity status of each function is stated in its docstring; all are pinned by
``tests/test_oracle_pins.py`` (closed forms, library routines, invariants).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16 = 0
BF16 = 1
_DT = {"fp16": F16, "f16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}

_lib = None


def build(force=False):
    """Compile attn_oracle.c with gcc into liboracle.so (seconds)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-Wall", "-shared",
                               "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load(path=None):
    global _lib
    if _lib is None or path is not None:
        if path is None:
            build()
        lib = ctypes.CDLL(path or _LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_paged_attention.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, D, I, I, P,
                                               P]
        lib.oracle_paged_attention.restype = I
        lib.oracle_dense_attention.argtypes = [I, I, I, I, I, I, P, P, P, D, I, I, P, P]
        lib.oracle_dense_attention.restype = I
        lib.oracle_paged_split_partials.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, D, I, I,
                                                    I, I, I, P, P]
        lib.oracle_paged_split_partials.restype = I
        lib.oracle_dense_split_partials.argtypes = [I, I, I, I, I, I, P, P, P, D, I, I, I, I, I, P,
                                                    P]
        lib.oracle_dense_split_partials.restype = I
        lib.oracle_combine.argtypes = [I, I, I, P, P, P, P]
        lib.oracle_combine.restype = None
        lib.oracle_decode_scalar.argtypes = [ctypes.c_uint16, I]
        lib.oracle_decode_scalar.restype = D
        if path is not None:
            return lib
        _lib = lib
    return _lib


class use_library:
    """Context manager: route every oracle call through another build of
    attn_oracle.c (used by the test that plants mistakes in the oracle)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _dt(dtype):
    if isinstance(dtype, int):
        return dtype
    return _DT[str(dtype).replace("torch.", "")]


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle takes raw 16-bit patterns as uint16, got %s" % a.dtype)
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


MAX_THREADS = 16  # worker threads at most: one GPU's share of a measurement host's cores


def host_cpus():
    """CPUs this process may run on (the nproc count)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def default_threads():
    """Worker threads: every CPU this process may use, at most MAX_THREADS."""
    return max(1, min(MAX_THREADS, host_cpus()))


def decode16(bits, dtype):
    """Exact float64 value of each 16-bit pattern (oracle's own decoder)."""
    lib = _load()
    dt = _dt(dtype)
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.empty(flat.shape, dtype=np.float64)
    for i, x in enumerate(flat):
        out[i] = lib.oracle_decode_scalar(int(x), dt)
    return out.reshape(np.shape(bits))


def paged_attention(q, k_cache, v_cache, block_table, cache_seqlens, dtype, scale=None,
                    nthreads=None, causal=False):
    """Exact attention over a paged KV cache (two-pass softmax, float64).

    causal: query i of qlen sees keys j <= L - qlen + i (bottom-right).

    q: uint16 [B, qlen, Hq, d]; k_cache, v_cache: uint16 [pages, page, Hkv, d];
    block_table: int32 [B, max_pages]; cache_seqlens: int32 [B].
    Returns (out float64 [B, qlen, Hq, d], lse float64 [B, Hq, qlen]).
    scale defaults to 1/sqrt(d).
    """
    lib = _load()
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    bt, sl = _i32(block_table), _i32(cache_seqlens)
    B, qlen, hq, d = q.shape
    _, page, hkv, d2 = kc.shape
    assert d2 == d and vc.shape == kc.shape and bt.shape[0] == B and sl.shape == (B,)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, qlen, hq, d), dtype=np.float64)
    lse = np.zeros((B, hq, qlen), dtype=np.float64)
    rc = lib.oracle_paged_attention(B, qlen, hq, hkv, d, page, bt.shape[1], _dt(dtype), _p(q),
                                    _p(kc), _p(vc), _p(bt), _p(sl), float(scale), int(causal),
                                    nthreads or default_threads(), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_paged_attention rejected the shape")
    return out, lse


def dense_attention(q, k, v, dtype, scale=None, nthreads=None, causal=False):
    """Exact attention, dense K/V (two-pass softmax, float64).

    q: uint16 [Hq, qlen, d]; k, v: uint16 [Hkv, kvlen, d].
    Returns (out float64 [Hq, qlen, d], lse float64 [Hq, qlen]).
    """
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    hq, qlen, d = q.shape
    hkv, kvlen, d2 = k.shape
    assert d2 == d and v.shape == k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((hq, qlen, d), dtype=np.float64)
    lse = np.zeros((hq, qlen), dtype=np.float64)
    rc = lib.oracle_dense_attention(hq, hkv, qlen, kvlen, d, _dt(dtype), _p(q), _p(k), _p(v),
                                    float(scale), int(causal), nthreads or default_threads(),
                                    _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_dense_attention rejected the shape")
    return out, lse


def split_keys_for(max_len, num_splits, granule=16):
    """One split length for a batch: C = granule * ceil(ceil(max_len/granule)/S)
    (at least one granule)."""
    units = -(-max(int(max_len), 0) // granule)
    return granule * max(1, -(-units // num_splits))


def paged_split_partials(q, k_cache, v_cache, block_table, cache_seqlens, dtype, num_splits,
                         split_keys, block=16, scale=None, nthreads=None, causal=False):
    """Per-split partials via the online-softmax recurrence (float64).

    Split s of a sequence with L keys covers keys [s*C, (s+1)*C) clipped to
    [0, L), C = split_keys (S*C must reach every L).  Returns
    (o_part [S, B*qlen*Hq, d], lse_part [S, B*qlen*Hq]) with rows
    n = (b*qlen + i)*Hq + hq; empty splits give zeros and -inf.
    """
    lib = _load()
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    bt, sl = _i32(block_table), _i32(cache_seqlens)
    B, qlen, hq, d = q.shape
    _, page, hkv, _ = kc.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n = B * qlen * hq
    o = np.zeros((num_splits, n, d), dtype=np.float64)
    l = np.zeros((num_splits, n), dtype=np.float64)
    rc = lib.oracle_paged_split_partials(B, qlen, hq, hkv, d, page, bt.shape[1], _dt(dtype),
                                         _p(q), _p(kc), _p(vc), _p(bt), _p(sl), float(scale),
                                         int(causal), num_splits, split_keys, block,
                                         nthreads or default_threads(), _p(o), _p(l))
    if rc != 0:
        raise ValueError("oracle_paged_split_partials rejected the shape")
    return o, l


def dense_split_partials(q, k, v, dtype, num_splits, split_keys, block=16, scale=None,
                         nthreads=None, causal=False):
    """Dense-layout counterpart of paged_split_partials; rows n = hq*qlen + i."""
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    hq, qlen, d = q.shape
    hkv, kvlen, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n = hq * qlen
    o = np.zeros((num_splits, n, d), dtype=np.float64)
    l = np.zeros((num_splits, n), dtype=np.float64)
    rc = lib.oracle_dense_split_partials(hq, hkv, qlen, kvlen, d, _dt(dtype), _p(q), _p(k), _p(v),
                                         float(scale), int(causal), num_splits, split_keys, block,
                                         nthreads or default_threads(), _p(o), _p(l))
    if rc != 0:
        raise ValueError("oracle_dense_split_partials rejected the shape")
    return o, l


def combine(o_part, lse_part):
    """Max-shifted log-sum-exp merge of S partials.

    o_part [S, n, d], lse_part [S, n] (float64) -> (out [n, d], lse [n]).
    """
    lib = _load()
    o = np.ascontiguousarray(o_part, dtype=np.float64)
    l = np.ascontiguousarray(lse_part, dtype=np.float64)
    S, n, d = o.shape
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    lib.oracle_combine(S, n, d, _p(o), _p(l), _p(out), _p(lse))
    return out, lse
