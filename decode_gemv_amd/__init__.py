"""MI355X (gfx950) GEMV over losslessly entropy-coded LLM weights.

The product is the C-ABI library liblw.so (include/lw.h); this package holds
its HIP/C++ sources (csrc/), the build script and a thin ctypes binding (lw)
whose functions carry the C names.
"""
from .lw import *  # noqa: F401,F403
from .lw import Bundle, DevBundle, LwError, header_functions, lib, upload  # noqa: F401
