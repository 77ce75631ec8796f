"""Contextually sparse gated-FFN decode step for AMD Instinct MI355X (gfx950).

The compute lives in ``libsparse_ffn.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/sparse_ffn.h``). ``binding`` is the thin ctypes layer over it;
``inputs`` holds the seeded synthetic workloads. Importing this package loads neither:
``from contextual_activation_sparsity_amd import binding`` loads the library and fails
loudly if it has not been built.
"""

__all__ = ["binding", "inputs"]
