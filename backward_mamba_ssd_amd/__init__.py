"""MI355X-native Mamba-2 selective SSM recurrence.

The compute lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``); ``backward_mamba_ssd_amd.ssm`` is its thin ctypes binding and
``backward_mamba_ssd_amd.inputs`` the seeded synthetic-input generators.  Nothing
is imported eagerly here so the generators load without the GPU library.
"""
__all__ = ["ssm", "inputs"]
