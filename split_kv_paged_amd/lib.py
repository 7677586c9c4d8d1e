"""ctypes view of the C ABI in include/attn_decode.h (argument marshalling only).

Loading fails loudly when libattn_decode.so has not been built: there is no
other implementation to fall back to.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_decode.so")

ATTN_OK = 0
STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ARG", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_ALIGN", 7: "ATTN_ERR_HIP",
    8: "ATTN_ERR_DATA",
}
FP16, BF16 = 0, 1

# every symbol the header declares
EXPORTS = (
    "attn_decode_plan", "attn_decode_fwd", "attn_decode_fwd_noalloc", "attn_decode_kvcache_fwd",
    "attn_decode_varlen_fwd",
    "attn_dense_plan", "attn_dense_fwd",
    "attn_combine_fwd", "attn_check_paged_inputs", "attn_check_kvcache_inputs",
    "attn_last_plan", "attn_status_str",
    "attn_abi_version",
)


class DecodeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_heads_q", "num_heads_kv", "head_dim", "page_size",
        "max_pages_per_seq", "max_seqlen_k", "dtype")] + [("sum_seqlen_k", ctypes.c_int64)]


class DenseShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_heads_q", "num_heads_kv", "q_len", "kv_len", "head_dim", "dtype")]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_splits", "pack_gqa", "rows_per_unit", "rows_per_block", "row_blocks", "units",
        "grid", "split_granule", "num_cus", "combine", "kernel", "split_keys",
        "heads_per_row", "extra_blocks")] + [
        ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class AttnError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(code, code), text))
        self.code = code
        self.status = STATUS.get(code, str(code))


_lib = None


def load():
    """The built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libattn_decode.so is not built (expected at %s); run "
            "`python -m split_kv_paged_amd.build` or __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    I64 = ctypes.c_int64
    sd, sn, pl = ctypes.POINTER(DecodeShape), ctypes.POINTER(DenseShape), ctypes.POINTER(Plan)
    sig = {
        "attn_decode_plan": ([sd, I, I, I, pl], I),
        "attn_decode_fwd": ([sd, P, P, P, P, P, I, I, F, P, P, P, Z, P], I),
        "attn_decode_fwd_noalloc": ([sd, P, P, P, P, P, I, I, F, P, P, P], I),
        "attn_decode_kvcache_fwd": ([sd, P, P, P, P, P, P, P, I, I, I, I, F, P, P, P, Z, P], I),
        "attn_decode_varlen_fwd": ([sd, P, P, P, P, P, P, I, P, P, I, I, I, F, P, P, P, Z, P], I),
        "attn_dense_plan": ([sn, I, I, pl], I),
        "attn_dense_fwd": ([sn, P, P, P, I, F, P, P, P, Z, P], I),
        "attn_combine_fwd": ([I, I, I, I, I, I, P, P, P, P, P], I),
        "attn_check_paged_inputs": ([sd, P, P, I64, ctypes.POINTER(ctypes.c_int32)], I),
        "attn_check_kvcache_inputs": ([sd, P, P, I64, I, ctypes.POINTER(ctypes.c_int32)], I),
        "attn_last_plan": ([pl], I),
        "attn_status_str": ([I], ctypes.c_char_p),
        "attn_abi_version": ([], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(fn, code):
    if code != ATTN_OK:
        text = load().attn_status_str(code).decode()
        raise AttnError(fn, code, text)
