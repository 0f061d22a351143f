"""Exact fused attention forward pass for AMD MI355X (gfx950).

The compute path is the HIP library ``libattn.so`` built from ``csrc/``; the
module ``exact_attention_47_amd.attn`` is a thin ctypes binding with the same
entry points. Nothing is imported here, so that the seeded input generators
(``exact_attention_47_amd.inputs``) can be used on machines without a GPU and
without the built library.
"""
