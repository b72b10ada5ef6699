"""MI355X-native SATA (symmetry-aware Taylor approximation) attention.

The computation lives in libsata.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/sata.h); ``constant_cost_attention_amd.sata`` is its
ctypes binding.  Import the binding explicitly:

    from constant_cost_attention_amd import sata
"""
__all__ = ["sata", "build"]
