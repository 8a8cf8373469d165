"""YOCO cross-decoder hot path on MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI declared in
``include/yoco.h`` (``libyoco.so``, built in this directory).  Submodules:
``binding`` loads the library with ctypes and exposes its calls; ``synth``
draws seeded synthetic workloads.  Importing the package itself loads
nothing, so the input generators work on machines without a GPU.
"""
