"""libmha: the Transformer's multi-head attention sublayer on MI355X (gfx950).

The compute lives in the C-ABI shared library ``libmha.so`` (hand-written HIP
kernels, declared in ``include/mha.h``).  ``transformer_head_scaled_amd.libmha``
is the thin ctypes binding with the same names; ``synth`` draws the seeded
synthetic inputs.
"""
