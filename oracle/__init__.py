"""fp64 CPU oracle for the multi-head attention sublayer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
loads anything from this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
header, table or helper with the HIP library, and it never imports the
product package.

Every function here is the plain definition the pages give, written in
float64 numpy with no blocking, fusion or reordering.  Sources, cited by page
title and section:

* nickwang.xyz, "Lire « Attention Is All You Need » : l'article original du
  Transformer" -- sections "Attention par produit scalaire mis à l'échelle"
  (paper §3.2.1, eq. (1) and its footnote), "Trois usages de l'attention dans
  le modèle" (paper §3.2.3) and "Attention multi-têtes : huit têtes de 64
  dimensions" (paper §3.2.2).
* agi-iri.ru, "Attention Is All You Need (на русском)" -- §3.2.1 "Scaled
  Dot-Product Attention" (the causal mask allows positions up to and
  including the current one) and §3.2.2 "Multi-Head Attention".
* ml-canon.vercel.app, "32 Transformer" -- "PyTorch: реализация" (the
  (..., seq, d_k) layout, the head split by columns, weights multiplied on
  the right).
* nickwang.xyz, the section on the encoder and decoder stacks (paper §3.1):
  the residual connection and layer normalisation around each sub-layer,
  LayerNorm(x + Sublayer(x)) (``layernorm.py``; LayerNorm itself is the
  standard definition, which the pages do not write out).

Parity status: every public function is pinned by tests under ``tests/``
(``test_oracle_pins.py`` and ``test_oracle_mutants.py``); none is "parity
unpinned".  The one printed number that cannot be reproduced, the worked
example's output vector o₁ on the nickwang.xyz page, is unpinned because the
page does not print the value vectors it was computed from; it does not
belong to any function here.
"""

from .attention import (  # noqa: F401
    MASK_CAUSAL,
    MASK_NONE,
    attention_head,
    band,
    mha,
    scores,
    sdpa,
    softmax_rows,
    visible,
    weighted_sum,
)
from .layernorm import add_norm, layer_norm, mha_add_norm  # noqa: F401
