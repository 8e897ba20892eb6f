"""Block-sparse attention over routed tiles, in float64 (test infrastructure only).

Sources (web pages):
- "H3 SLA Attention" node page, "How it works" and "The inputs that matter":
  each query block attends only its selected key blocks plus the protected
  [text | cond | audio] blocks; unselected blocks get a hard zero (the tail
  term is an off-by-default option and is not part of this path).
- "Flash Partitions for H3 native temporal alignment", section 1: the same
  score rule as dense TARA inside the attended tiles.
"""
from __future__ import annotations

import numpy as np

from .tara import tara_bias, _softmax_rows


def block_sparse_block(q_h, k_h, v_h, seg, t, params, scale, block_size, prot, tiles_row, qb):
    """Output rows of query block ``qb`` for one head.

    q_h, k_h, v_h: [n, d] float64. ``prot``: protected block indices;
    ``tiles_row``: routed block indices of this (head, query block); entries
    outside the sequence's blocks are ignored. The keys are the rows of the set
    of protected and routed blocks (a block listed twice counts once); the
    softmax runs over those keys only, with the dense TARA score
    s_ij = scale * q_i . k_j - p_ij. Returns (o [rows, d], lse [rows]).
    """
    n = q_h.shape[0]
    nb = (n + block_size - 1) // block_size
    lo, hi = qb * block_size, min(n, (qb + 1) * block_size)
    blocks = sorted({int(b) for b in list(prot) + list(tiles_row) if 0 <= int(b) < nb})
    if not blocks:
        return np.zeros((hi - lo, q_h.shape[1])), np.full(hi - lo, -np.inf)
    keys = np.concatenate([np.arange(b * block_size, min(n, (b + 1) * block_size))
                           for b in blocks])
    s = scale * (q_h[lo:hi] @ k_h[keys].T) - tara_bias(seg[lo:hi], t[lo:hi], seg[keys],
                                                        t[keys], params)
    return _softmax_rows(s, v_h[keys])


def block_sparse(q, k, v, seg, t, params, scale, block_size, prot, tiles, heads=None,
                 qblocks=None):
    """Block-sparse outputs for the selected heads and query blocks.

    q, k, v: [n, H, d] float64; tiles: [H, nqb, k_sel]. Returns
    {(h, qb): (o_rows, lse_rows)} for every requested pair.
    """
    n, H, d = q.shape
    nqb = (n + block_size - 1) // block_size
    heads = range(H) if heads is None else heads
    qblocks = range(nqb) if qblocks is None else qblocks
    out = {}
    for h in heads:
        qh = np.ascontiguousarray(q[:, h, :])
        kh = np.ascontiguousarray(k[:, h, :])
        vh = np.ascontiguousarray(v[:, h, :])
        for qb in qblocks:
            out[(h, qb)] = block_sparse_block(qh, kh, vh, seg, t, params, scale, block_size,
                                              prot, tiles[h][qb], qb)
    return out
