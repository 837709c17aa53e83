"""Exact tiled softmax attention for MI355X (gfx950): HIP kernels behind a C ABI.

libfa355 (built in-tree by ``build.py``) holds the forward, the three-stage
backward, the packed variable-length forms, the persistent longest-first
forward, split-KV decoding with grouped-query packing, and the FP8 forward with
a Hadamard rotation; ``fa355`` is its ctypes binding, ``workloads`` the seeded
synthetic inputs and ``accounting`` the FLOP and byte counts.
"""
