"""Head-wise sparse attention (RTPurbo) on AMD Instinct MI355X (gfx950).

``head_wise_sparse_amd.rtp``       ctypes binding of the C-ABI library ``librtp.so``
``head_wise_sparse_amd.workloads`` seeded synthetic inputs (no method arithmetic)
"""
__all__ = ["rtp", "workloads"]
