"""MI355X-native DCNv4 spatial aggregation (forward and backward).

The operator itself lives in the HIP/C library ``libdcnv4.so`` (gfx950).
``dynamic_sparse_vision_amd.dcnv4`` is the thin ctypes binding over its C ABI;
``synth`` and ``workloads`` describe the seeded synthetic inputs.
"""
__all__ = ["dcnv4", "synth", "workloads"]
