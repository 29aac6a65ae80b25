"""Chunk-swizzled AllGather-GEMM, GEMM-ReduceScatter and AG-MoE for AMD MI355X.

The compute path is the C-ABI library ``libtlc.so`` (HIP kernels for gfx950,
declared in ``include/tlc.h``); ``tile_level_communication_amd.tlc`` is its
ctypes binding and ``tile_level_communication_amd.workloads`` sets up device
buffers for the three operations.  PyTorch only provides device memory and
streams.
"""
__all__ = ["tlc", "workloads", "build"]
