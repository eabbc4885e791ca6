"""Unified draft/verify decode attention with PillarAttn top-K for MI355X (gfx950).

The compute path is the HIP library ``libspa.so`` behind the C ABI declared in
``include/spa.h``; ``binding`` marshals PyTorch device tensors into it.
"""
