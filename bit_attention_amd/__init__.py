"""MI355X-native microscaling-FP4 attention forward (SageAttention3-style) for gfx950.

The compute path is the C-ABI library ``libsage_fp4.so`` (hand-written HIP kernels); the Python
binding in :mod:`bit_attention_amd.binding` only marshals arguments. Nothing is loaded at import
time.
"""
