"""The oracle: a plain fp64 CPU implementation of the paged-attention forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything in this package;
the HIP library and its Python binding never do.
"""
