"""split_kv_paged_amd: exact split-KV decode / small-query attention for MI355X (gfx950).

The compute path is a C-ABI shared library (``include/attn_decode.h``) built
from hand-written HIP kernels under ``csrc/``.  This package only marshals
arguments to it: ``api`` takes torch tensors (device memory, streams) and
calls the library; nothing here computes attention.

Submodules are imported lazily so that ``workloads`` (seeded synthetic
inputs, numpy only) can be used without loading the GPU library.
"""
import importlib

__all__ = ["api", "lib", "workloads", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
