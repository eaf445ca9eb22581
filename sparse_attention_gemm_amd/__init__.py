"""MI355X (gfx950) implementation of the DeepSeek Sparse Attention hot path.

The compute path is libdsa.so (HIP kernels behind the C ABI in include/dsa.h);
``sparse_attention_gemm_amd.dsa`` is its ctypes binding.  Build it with
``python -m sparse_attention_gemm_amd.build``.
"""
__all__ = ["dsa", "build"]
