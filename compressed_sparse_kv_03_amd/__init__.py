"""MI355X-native hybrid compressed attention (CSA + HCA).

The compute path is libcskv.so (HIP kernels for gfx950, C ABI in
include/cskv.h); `native` is its ctypes binding and `synth` holds the seeded
synthetic-input generators. Nothing is imported eagerly, so the generators
can be used where the library has not been built.
"""
__all__ = ["native", "synth", "configs"]
