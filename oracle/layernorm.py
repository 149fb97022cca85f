"""Residual connection and layer normalisation ("Add & Norm") in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

nickwang.xyz, "Lire « Attention Is All You Need »", the section on the two
stacks (paper §3.1): every sub-layer is wrapped by a residual connection
followed by layer normalisation, so a sub-layer's output is
LayerNorm(x + Sublayer(x)) -- normalisation after the addition (Post-Norm),
all sub-layers producing d_model features so that the addition is defined.
The "Add & Norm" boxes of the architecture figure on the same page are this
step.  agi-iri.ru and ml-canon.vercel.app ("32 Transformer") describe the
same block: attention, then residual + LayerNorm.

The pages do not write LayerNorm out.  The reading taken here is the
standard layer normalisation: over the d_model features of ONE position,
the mean mu and the mean squared deviation sigma^2 (divided by d_model, not
d_model - 1), then gamma * (z - mu) / sqrt(sigma^2 + eps) + beta with a
per-feature gain gamma and bias beta and a small eps > 0 chosen by the
caller.  Inputs are upcast exactly to float64; nothing is rounded.
"""

import numpy as np

from .attention import MASK_NONE, mha


def layer_norm(z, gamma, beta, eps):
    """Layer normalisation of z [..., d] over its last axis, float64."""
    z = np.asarray(z, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    dev = z - mu
    var = (dev * dev).mean(axis=-1, keepdims=True)
    return gamma * dev / np.sqrt(var + float(eps)) + beta


def add_norm(x, sub, gamma, beta, eps):
    """LayerNorm(x + sub): the residual addition, then layer normalisation."""
    z = np.asarray(x, dtype=np.float64) + np.asarray(sub, dtype=np.float64)
    return layer_norm(z, gamma, beta, eps)


def mha_add_norm(x_q, x_kv, Wq, Wk, Wv, Wo, gamma, beta, eps, h, mask_kind=MASK_NONE,
                 kv_lens=None):
    """The attention sub-layer with its Add & Norm:
    LayerNorm(x_q + MultiHead(x_q, x_kv, x_kv)).  The residual is the
    sub-layer's query-side input (for encoder-decoder attention, the
    decoder stream)."""
    return add_norm(x_q, mha(x_q, x_kv, Wq, Wk, Wv, Wo, h, mask_kind, kv_lens), gamma, beta, eps)
