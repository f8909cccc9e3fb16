"""Stem block-sparse causal prefill on MI355X (gfx950).

The compute path lives in libstem.so (HIP kernels behind the C ABI of
include/stem.h); ``block_sparse_causal_amd.stem`` is its Python binding and
``block_sparse_causal_amd.synthetic`` draws seeded inputs.  The library is
loaded on first use; nothing here falls back to a CPU implementation.
"""
