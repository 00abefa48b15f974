"""Chunkwise causal linear attention on MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``liblinattn.so`` (built from ``csrc/``); this package holds
the ctypes binding (``binding``), the seeded input generators (``inputs``) and the
named workloads (``workloads``). Importing the package does not load the library;
the first call through ``binding`` does, and fails loudly if it is not built.
"""
__all__ = ["binding", "inputs", "workloads"]
