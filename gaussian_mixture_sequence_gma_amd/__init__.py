"""MI355X-native Gaussian Mixture Attention (GMA) forward.

The computation lives in libgma.so (HIP kernels for gfx950 behind the C ABI of
include/gma.h).  ``binding`` exposes the C entry points by name, ``api`` adds
shape handling and torch allocation, ``inputs`` draws seeded synthetic inputs.
Submodules are imported on demand so that ``inputs`` works without a GPU or a
built library.
"""
__all__ = ["api", "binding", "inputs", "build"]
