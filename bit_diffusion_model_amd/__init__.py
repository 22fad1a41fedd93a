"""MI355X (gfx950) SVDQuant W4A4 + low-rank linear layer.

The compute lives in a C-ABI shared library (``libsvdq.so``, HIP kernels for gfx950
plus host-side packing); ``bit_diffusion_model_amd.svdq`` is the thin ctypes binding
over it.  ``bit_diffusion_model_amd.workloads`` generates the seeded synthetic inputs.
"""
__all__ = ["workloads"]
