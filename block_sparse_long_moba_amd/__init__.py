"""MoBA (Mixture of Block Attention) forward pass for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmoba.so`` built from ``csrc/``; the
Python side (``moba``) only marshals arguments to its C ABI.
"""
__all__ = ["synth"]
