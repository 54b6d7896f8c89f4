"""MI355X (gfx950) GEMV over losslessly entropy-coded LLM weights.

The product is the C-ABI library liblw.so (include/lw.h); this package holds
its HIP/C++ sources (csrc/), the build script and a thin ctypes binding (lw)
whose functions carry the C names.

The binding loads on first use of any of its names (``decode_gemv_amd.lw_gemv``
and so on), so that the build script can run before liblw.so exists; if the
library is missing, that first use raises ImportError.
"""
from __future__ import annotations


import importlib


def __getattr__(name):
    if name.startswith("__"):
        raise AttributeError(name)
    if name in ("lw", "build"):          # submodules (``from decode_gemv_amd import build``)
        return importlib.import_module(__name__ + "." + name)
    lw = importlib.import_module(__name__ + ".lw")
    try:
        return getattr(lw, name)
    except AttributeError:
        raise AttributeError(f"module 'decode_gemv_amd' has no attribute {name!r}") from None
