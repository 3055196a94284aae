"""MI355X-native learned block-compressed attention (LBCA / HCA / CSA).

The compute lives in ``liblbca.so`` (hand-written HIP for gfx950 behind the C-ABI
declared in ``include/lbca.h``).  ``block_compressed_kv_amd.lbca`` is the thin
ctypes binding; ``block_compressed_kv_amd.synth`` holds the seeded synthetic
input generators.  Importing this package loads nothing: the library is opened
on first use of the binding, and raises if it has not been built.
"""

__all__ = ["lbca", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
