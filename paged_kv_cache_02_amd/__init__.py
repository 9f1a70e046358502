"""Attention over a paged KV cache for AMD Instinct MI355X (gfx950).

The computation lives in ``libpkv.so`` (hand-written HIP kernels behind the C
ABI of ``include/pkv.h``); ``paged_kv_cache_02_amd.pkv`` is its ctypes
binding.  Build the library with ``python -m paged_kv_cache_02_amd.build``.
"""

import importlib

__all__ = ["pkv"]


def __getattr__(name):
    if name == "pkv":
        return importlib.import_module(__name__ + ".pkv")
    raise AttributeError(name)
