"""MI355X-native expert-ID matmul (matmul_id) for mixture-of-experts layers.

The compute lives in libeidm.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/eidm.h).  `binding` is a thin ctypes layer over that ABI that
takes torch tensors for device memory and streams; `workloads` draws the
seeded synthetic inputs.  Importing the package loads nothing.
"""
__all__ = ["binding", "workloads", "build"]
