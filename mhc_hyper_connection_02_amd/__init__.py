"""MI355X-native fused mHC boundary: HIP kernels for gfx950 behind a C ABI.

The compute runs in ``libmhc_amd.so`` (built from ``csrc/``); the Python side
only marshals torch tensors into its entry points. Importing the package does
not load the library; the first call into :mod:`.binding` does, and fails
loudly if it is missing.
"""

__all__ = ["binding", "synth"]
