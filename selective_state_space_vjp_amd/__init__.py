"""MI355X-native backward (VJP) of the selective state-space scan.

The compute lives in ``libssmvjp.so`` (hand-written HIP for gfx950, C ABI in
``include/ssmvjp.h``); :mod:`selective_state_space_vjp_amd.binding` marshals
torch tensors into that ABI.  Nothing here computes on the CPU.
"""
__all__ = ["binding", "synth"]
