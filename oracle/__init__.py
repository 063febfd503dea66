"""fp64 CPU oracle for the MSA forward pass -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``block_sparse_long_bk_amd`` and imports nothing from it.
"""
