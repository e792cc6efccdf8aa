"""DSpark semi-autoregressive drafting hot path for AMD MI355X (gfx950).

The compute path is the C-ABI library `libdspark.so` built from hand-written HIP
kernels (see `semi_autoregressive_drafting_amd.dspark` for the Python binding).
Importing this package does not load the library; `synth` (seeded inputs) is
usable on any host.
"""
__all__ = ["synth", "dspark"]
