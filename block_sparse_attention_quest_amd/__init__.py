"""MI355X-native hot path of Rectified Sparse Attention (ReSA).

The compute lives in ``libresa.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/resa.h``). The Python side only marshals arguments:
``block_sparse_attention_quest_amd.resa`` exposes the same four calls,
``resa_update_descriptors``, ``resa_select_blocks``, ``resa_sparse_decode`` and
``resa_rectify``, taking torch tensors for device memory and the current stream.

Importing the package does not load the library; the first call does, and it
raises if the library has not been built.
"""

__all__ = ["resa", "workloads"]
