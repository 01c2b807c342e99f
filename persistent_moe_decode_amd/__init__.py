"""Persistent MoE decode megakernel for MI355X: Python side of the C ABI.

``mk`` is the ctypes binding of ``libmk.so`` (include/mk.h); ``runtime``
allocates the model's device buffers with PyTorch and drives decode steps
through the binding.  Nothing is imported eagerly, so the seeded input
generator and the oracle never pull in the GPU path.
"""
__all__ = ["mk", "runtime", "build"]
