"""CSA2 (Compressed Sparse Attention 2) hot path for AMD Instinct MI355X.

The compute lives in ``libcsa2.so`` (hand-written gfx950 HIP kernels behind
the C ABI of include/csa2.h); ``api`` marshals torch tensors into it and
``gen`` draws seeded synthetic inputs.  Importing the package does not load
the library; the first call does, and fails loudly if it is not built.
"""
__all__ = ["api", "gen", "build"]
