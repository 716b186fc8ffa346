"""ConvRot W8A8 INT8 linear for AMD Instinct MI355X (gfx950).

The HIP kernels and the C ABI live in ``libconvrot.so`` (``include/convrot.h``);
``w8a8_int8_rotated_amd.convrot`` is its Python binding and
``w8a8_int8_rotated_amd.workloads`` the seeded synthetic inputs.
"""
__all__ = ["convrot", "workloads", "build"]
