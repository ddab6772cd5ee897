"""GPT-2 training step (forward, backward, AdamW) on MI355X (gfx950).

The compute lives in a C-ABI shared library built from csrc/ (hand-written
HIP kernels); `gpt2` is its thin ctypes binding.  `synth` holds the seeded
input generators.  The binding is imported lazily so that the input
generators can be used on machines without the built library.
"""
import importlib

__all__ = ["gpt2", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
