"""MI355X-native NF4-style 4-bit weight-only linear layer.

The compute lives in ``libnf4.so`` (hand-written HIP for gfx950 behind a C
ABI, declared in ``include/nf4.h``); :mod:`bit_weight_only_amd.nf4` is the thin
ctypes binding with the same entry-point names.  Nothing is loaded at import
time, so ``import bit_weight_only_amd.synth`` works without the library.
"""
__all__ = ["nf4", "synth"]
