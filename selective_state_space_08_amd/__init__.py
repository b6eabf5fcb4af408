"""MI355X-native Mamba-2 selective state-space (SSD) layer.

The compute lives in ``libssd.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/ssd.h``).  ``selective_state_space_08_amd.ssd``
is the thin ctypes binding; importing this package itself loads nothing.
"""
__all__ = ["ssd", "synth", "workloads"]
