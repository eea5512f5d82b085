"""MI355X-native fused MoE router: score function + top-k selection, its
backward, and the aux-loss score variant, as hand-written HIP kernels for
gfx950 behind a C-ABI library (``include/router.h``).

Importing the package loads nothing; the HIP library is loaded on first use
by :mod:`score_function_top_amd.router`, which raises if it is not built.
"""

__all__ = ["router", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
