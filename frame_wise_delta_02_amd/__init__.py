"""MI355X-native Video Delta Attention (VDA) forward pass.

The compute lives in hand-written HIP kernels for gfx950 behind a C ABI
(``include/vdn_vda.h``, built into ``libvdn_vda.so`` next to this file).
``binding`` marshals torch tensors into that ABI; ``synth`` draws the seeded
synthetic workloads.  Importing the package loads nothing native: the library
is opened on first use and a missing build is an error, never a fallback.
"""
