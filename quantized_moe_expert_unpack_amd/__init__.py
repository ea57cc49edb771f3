"""Affine group-quantized mixture-of-experts FFN step for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C-ABI library
``libmoeq.so`` (header ``include/moeq.h``); ``quantized_moe_expert_unpack_amd.moeq``
is the thin ctypes binding over it.  ``synth`` draws seeded synthetic inputs.
Importing the package does not load the library: the binding loads it on first
use and raises if it is missing.
"""

__all__ = ["moeq", "synth"]
