"""MI355X-native Multi-head Latent Attention layer (Kimi-K2 dimensions).

The compute lives in a C-ABI shared library (`libmla.so`, HIP kernels for gfx950) declared in
`include/mla.h`. `binding` is a thin ctypes layer over it; `synth` generates seeded inputs.
Importing this package does not load the library; `binding.lib()` does, and raises if the
library has not been built.
"""
