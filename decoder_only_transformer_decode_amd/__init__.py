"""MI355X-native decode step of a Llama-family decoder-only transformer.

The compute path is the HIP library ``libdtd.so`` (C ABI declared in include/dtd.h);
``dtd`` is its thin ctypes binding and ``synth`` builds seeded synthetic inputs.
Importing the package loads nothing; ``dtd.load()`` opens the library.
"""
__all__ = ["dtd", "synth"]
