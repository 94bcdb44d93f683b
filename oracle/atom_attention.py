"""Float64 definition of window-batched sequence-local atom attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: page 1 ("NVIDIA BioNeMo escala modelagem biomolecular com context
parallelism ...", section "Atom sequence local attention eficiente"): AlphaFold3
restricts atom attention to local windows of 32 x 128, processed as a batch of
windows.  The page gives nothing else; the readings taken here (the plain
AlphaFold3 form) are:

  - atoms of a sequence are split into query blocks of 32 consecutive atoms;
    block w holds queries 32w .. 32w+31 (the last block may be partial);
  - block w attends to the 128 consecutive atoms centred on the block's
    centre 32w + 16, i.e. keys 32w - 48 .. 32w + 79; keys outside the sequence
    do not exist;
  - per head h:  s_ij = scale * q_i . k_j + bias[w, h, i - 32w, j - (32w - 48)],
    softmax over the block's existing, unmasked keys j, o_i = sum_j p_ij v_j;
  - an atom mask removes keys (not queries); a query whose window holds no
    existing unmasked key gets o_i = 0.
"""

from __future__ import annotations

import numpy as np

Q_BLOCK = 32
K_WINDOW = 128
K_OFFSET = Q_BLOCK // 2 - K_WINDOW // 2      # first key of block w is 32w + K_OFFSET = 32w - 48


def n_windows(n_atoms):
    return (n_atoms + Q_BLOCK - 1) // Q_BLOCK


def window_keys(w, n_atoms):
    """Key atom indices of query block w (K_WINDOW of them; some may lie
    outside [0, n_atoms))."""
    return np.arange(K_WINDOW) + Q_BLOCK * w + K_OFFSET


def window_attention(q, k, v, bias=None, mask=None, scale=None):
    """o[b, i, h, :] for q, k, v of shape [batch, n_atoms, heads, d].

    ``bias`` is [batch, n_windows, heads, 32, 128] (query row, key column of
    the window) or None; ``mask`` is [batch, n_atoms] (nonzero keeps the atom as
    a key) or None; ``scale`` defaults to 1 / sqrt(d).  Returns float64
    [batch, n_atoms, heads, d].
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    bsz, n, heads, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((bsz, n, heads, d))
    for w in range(n_windows(n)):
        qi = np.arange(Q_BLOCK * w, min(Q_BLOCK * (w + 1), n))
        kj = window_keys(w, n)
        exists = (kj >= 0) & (kj < n)
        kc = np.clip(kj, 0, n - 1)
        for b in range(bsz):
            keep = exists.copy()
            if mask is not None:
                keep &= np.asarray(mask)[b, kc] != 0
            if not keep.any():
                continue
            # [heads, |qi|, 128] logits, one matrix product per head
            s = scale * np.einsum("ihd,jhd->hij", q[b, qi], k[b, kc])
            if bias is not None:
                s = s + np.asarray(bias, dtype=np.float64)[b, w, :, :len(qi), :]
            s = np.where(keep[None, None, :], s, -np.inf)
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            out[b, qi] = np.einsum("hij,jhd->ihd", p, v[b, kc])
    return out
