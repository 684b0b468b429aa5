"""MI355X-native GDLA (Grouped Differential Latent Attention) forward pass.

The compute lives in the C-ABI HIP library libgdla.so (built from csrc/); the
Python side only marshals pointers, sizes and streams.  Importing the package
does not load the library; the first call does, and fails loudly if it is
missing.
"""
