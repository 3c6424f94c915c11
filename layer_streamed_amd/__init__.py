"""MI355X-native layer-streamed training step.

The compute lives in ``libmt.so`` (HIP for gfx950, C ABI declared in
``include/mt.h``).  ``layer_streamed_amd.mt`` is a thin ctypes binding over
it; importing this package does not load the library, so host-only helpers
(``metrics``) stay usable on machines without the build.
"""
import importlib

__all__ = ["mt", "metrics"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
