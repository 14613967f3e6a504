"""MI355X-native Compressed Sparse Attention (CSA) hot path.

The compute path is the HIP library ``libcsa.so`` (C ABI declared in
``include/csa.h``); :mod:`.binding` is a thin ctypes layer over it and
:mod:`.synth` generates seeded synthetic inputs. Importing this package does
not load the library; ``binding.lib()`` does, and fails loudly when it is
missing.
"""
__all__ = ["binding", "synth", "cache"]
