"""Attention-space KV-cache scoring and budgeted top-k for AMD MI355X (gfx950).

The compute path is libkvs.so (hand-written HIP kernels behind a C ABI, see
include/kvs.h); ``attention_space_retrieval_amd.kvs`` is its ctypes binding.
``workloads`` draws the seeded synthetic inputs.  Importing the package loads
nothing; the binding loads the library on first use.
"""
