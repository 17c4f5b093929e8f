"""Routed MoE expert FFN over frozen packed 4-bit experts, native to MI355X (gfx950).

The compute path is the HIP library ``csrc/libmoeq.so`` behind a C-ABI
(``include/moeq.h``); ``moeq`` is its thin Python binding.  Importing this package
does not load the library; the first call does, and fails loudly if it is missing.
"""
__all__ = ["synth", "moeq"]
