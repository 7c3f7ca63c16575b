"""PACK3D local-global attention over a packed 3D token volume, MI355X-native.

* ``geometry_aware_local_amd.pack3d`` - Python binding of ``libpack3d.so``
  (the HIP kernels behind the C ABI in ``include/pack3d.h``); importing it
  loads the library and fails if it has not been built.
* ``geometry_aware_local_amd.build`` - builds the library with hipcc for gfx950.
"""

__all__ = ["pack3d", "build"]
