"""BLASST skip-softmax attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libblasst.so`` (hand-written HIP kernels behind a C
ABI, ``include/blasst.h``). ``block_sparse_long_skip_amd.attention`` is a thin
ctypes binding over it; PyTorch supplies device memory and streams only.
``block_sparse_long_skip_amd.synth`` makes seeded synthetic inputs.

Importing the package does not load the native library; the first call into
``attention`` does, and raises if it is missing.
"""

__all__ = ["attention", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
