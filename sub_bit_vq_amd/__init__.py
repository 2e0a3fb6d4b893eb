"""libloopvq: LoopVQ sub-bit KV-cache decode attention and encoder for MI355X.

The compute lives in a C-ABI shared library (``libloopvq.so``, HIP for gfx950)
declared in ``include/loopvq.h``; :mod:`sub_bit_vq_amd.loopvq` is its thin
Python binding.  :mod:`sub_bit_vq_amd.synth` generates seeded synthetic
inputs.  Importing the package does not load the library; the first call
through the binding does, and raises if it is missing.
"""

__all__ = ["loopvq", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
