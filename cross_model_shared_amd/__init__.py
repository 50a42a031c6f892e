"""Shared-KV attention on MI355X (gfx950): a paged KV pool read once by N decoders.

The compute lives in libkvshare.so (hand-written HIP kernels behind a C ABI,
declared in include/kvshare.h); `binding` marshals torch tensors into it.
Importing the package does not load the library; `binding.load()` does, and
fails loudly when it is missing.
"""
__all__ = ["binding", "workload"]
