"""MI355X-native speculative-decoding verify step.

The compute lives in libvstep.so (HIP kernels for gfx950 behind the C ABI in
include/vstep.h); verification_step_amd.api is a thin ctypes binding over it.
"""
__all__ = ["api", "workloads", "build"]
