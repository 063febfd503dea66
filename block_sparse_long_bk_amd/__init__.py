"""MiniMax Sparse Attention (MSA) forward hot path for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels inside ``libmsa.so`` (C ABI,
declared in ``include/msa.h``).  This package is its thin Python binding:
``api`` marshals torch tensors into the C calls, ``inputs`` draws the seeded
synthetic workloads.  Importing the package loads nothing; the library is
loaded on the first call into ``api``.
"""

__all__ = ["api", "inputs"]


def __getattr__(name):
    if name in ("api", "inputs"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
