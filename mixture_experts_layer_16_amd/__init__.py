"""MI355X (gfx950) Mixture-of-Experts FFN layer forward pass.

The compute path is the HIP library ``libmoe.so`` (C ABI in include/moe.h);
``_lib`` is its thin ctypes binding.  Importing the binding requires the
library to be built (``python -m mixture_experts_layer_16_amd.build``).
"""
__version__ = "0.1.0"


def lib():
    """The ctypes binding (imports torch and loads libmoe.so)."""
    from . import _lib
    return _lib
