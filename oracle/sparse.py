"""Block-sparse attention over routed tiles, in float64 (test infrastructure only).

Sources (web pages):
- "H3 SLA Attention" node page, "How it works" and "The inputs that matter":
  each query block attends only its selected key blocks plus the protected
  [text | cond | audio] blocks; unselected blocks get a hard zero.
- same page, inputs table, tail_correction (off by default): instead of the
  hard zero, one pooled term stands in for every key block the top-k left out;
  its score reuses the routing's block means, so the extra work is a block mean
  of V and a small reduction.
- "Flash Partitions for H3 native temporal alignment", section 1: the same
  score rule as dense TARA inside the attended tiles.

Reading of the tail term (the page gives no formula): for query block qb and
its unrouted video tiles U, the term has logit
    L_tail = ln sum_{u in U} n_u * exp(scale * S[qb, u])
and value v_tail = (sum_u n_u exp(scale * S[qb, u]) vbar_u) / exp(L_tail), where
S is the router's float32 pooled score (unscaled q-mean . k-mean), n_u the rows of
tile u and vbar_u the mean of its V rows: every left-out key is stood in for by
its tile's centroids. It is one extra key of every row of the block; the TARA
penalty, like the routing, does not see it. With no unrouted tile it vanishes.

Block size: the same definitions hold for 32-, 64- and 128-row blocks ("H3 SLA
Attention", inputs table, block_size: the number of rows that share one key
selection; halving it doubles the block count and keeps the attention work).
Query blocks and key blocks have the same size.

Sink queries ("Per-layer attention config LoRAs", section "Experimental:
audio/text protection": with sink_queries = audio, attention of the audio
queries is computed without sparsity): a query block holding any row of a sink
segment attends every key of the sequence. Reading: the whole block is dense,
including its few non-sink rows at a segment boundary, and it has no tail term
since nothing is left out.
"""
from __future__ import annotations

import numpy as np

from .quant import int8_roundtrip
from .router import block_means_fp32, pooled_scores_fp32, router_plan
from .tara import tara_bias, _softmax_rows


def tail_terms(q32_h, k32_h, v_h, seg, protected_prefix_len, block_size, tiles_h, scale):
    """Tail terms of one head: (L_tail [nqb] natural log, v_tail [nqb, d] float64).

    q32_h, k32_h: [n, d] float32 input values (the router's pooled means and
    scores are float32 as in routing); v_h: [n, d] float64; tiles_h: [nqb, k]
    routed tiles (entries outside the video tiles are ignored). Query blocks with
    no unrouted video tile get (-inf, 0).
    """
    n = q32_h.shape[0]
    _, _, video, _ = router_plan(seg, protected_prefix_len, block_size, 0.0)
    qbar = block_means_fp32(q32_h, block_size)
    kbar = block_means_fp32(k32_h, block_size)
    vbar = np.stack([v_h[b * block_size:min(n, (b + 1) * block_size)].mean(axis=0)
                     for b in range(len(qbar))])
    counts = np.array([min(n, (b + 1) * block_size) - b * block_size for b in video],
                      dtype=np.float64)
    scores = pooled_scores_fp32(qbar, kbar[video]).astype(np.float64)
    nqb = len(qbar)
    lse = np.full(nqb, -np.inf)
    vt = np.zeros((nqb, v_h.shape[1]))
    for qb in range(nqb):
        routed = set(int(b) for b in tiles_h[qb])
        keep = np.array([int(b) not in routed for b in video], dtype=bool)
        if not keep.any():
            continue
        x = scale * scores[qb, keep] + np.log(counts[keep])
        m = x.max()
        w = np.exp(x - m)
        lse[qb] = m + np.log(w.sum())
        vt[qb] = (w[:, None] * vbar[video[keep]]).sum(axis=0) / w.sum()
    return lse, vt


def is_sink_block(seg, block_size, qb, sink_segments):
    """Whether query block ``qb`` holds a row of any segment in ``sink_segments``."""
    lo, hi = qb * block_size, min(len(seg), (qb + 1) * block_size)
    return any(int(x) in set(sink_segments) for x in np.asarray(seg)[lo:hi])


def block_sparse_block(q_h, k_h, v_h, seg, t, params, scale, block_size, prot, tiles_row, qb,
                       tail=None, sink_segments=()):
    """Output rows of query block ``qb`` for one head.

    q_h, k_h, v_h: [n, d] float64. ``prot``: protected block indices;
    ``tiles_row``: routed block indices of this (head, query block); entries
    outside the sequence's blocks are ignored. The keys are the rows of the set
    of protected and routed blocks (a block listed twice counts once); the
    softmax runs over those keys only, with the dense TARA score
    s_ij = scale * q_i . k_j - p_ij. ``tail`` = (L_tail, v_tail) of this block
    adds one key with logit L_tail and value v_tail to every row (see
    ``tail_terms``). A query block holding a row of a segment in
    ``sink_segments`` attends every key and takes no tail. Returns (o [rows, d],
    lse [rows]).
    """
    n = q_h.shape[0]
    nb = (n + block_size - 1) // block_size
    lo, hi = qb * block_size, min(n, (qb + 1) * block_size)
    if sink_segments and is_sink_block(seg, block_size, qb, sink_segments):
        blocks = list(range(nb))
        tail = None
    else:
        blocks = sorted({int(b) for b in list(prot) + list(tiles_row) if 0 <= int(b) < nb})
    keys = (np.concatenate([np.arange(b * block_size, min(n, (b + 1) * block_size))
                            for b in blocks]) if blocks else np.zeros(0, dtype=np.int64))
    s = scale * (q_h[lo:hi] @ k_h[keys].T) - tara_bias(seg[lo:hi], t[lo:hi], seg[keys],
                                                        t[keys], params)
    vals = v_h[keys]
    if tail is not None and np.isfinite(tail[0]):
        s = np.concatenate([s, np.full((hi - lo, 1), tail[0])], axis=1)
        vals = np.concatenate([vals, np.asarray(tail[1])[None, :]], axis=0)
    if s.shape[1] == 0:
        return np.zeros((hi - lo, q_h.shape[1])), np.full(hi - lo, -np.inf)
    return _softmax_rows(s, vals)


def block_sparse(q, k, v, seg, t, params, scale, block_size, prot, tiles, heads=None,
                 qblocks=None, tails=None, sink_segments=(), int8_qk=False):
    """Block-sparse outputs for the selected heads and query blocks.

    q, k, v: [n, H, d] float64; tiles: [H, nqb, k_sel]; tails: optional
    {h: (L_tail [nqb], v_tail [nqb, d])}; sink_segments: segment ids whose query
    blocks attend densely; int8_qk: scores from the per-token int8 images of q and
    k (oracle.quant; q and k must hold float32 values). Returns {(h, qb): (o_rows,
    lse_rows)} for every requested pair.
    """
    n, H, d = q.shape
    nqb = (n + block_size - 1) // block_size
    heads = range(H) if heads is None else heads
    qblocks = range(nqb) if qblocks is None else qblocks
    out = {}
    for h in heads:
        qh = np.ascontiguousarray(q[:, h, :])
        kh = np.ascontiguousarray(k[:, h, :])
        if int8_qk:
            qh, kh = int8_roundtrip(qh), int8_roundtrip(kh)
        vh = np.ascontiguousarray(v[:, h, :])
        for qb in qblocks:
            tail = None if tails is None else (tails[h][0][qb], tails[h][1][qb])
            out[(h, qb)] = block_sparse_block(qh, kh, vh, seg, t, params, scale, block_size,
                                              prot, tiles[h][qb], qb, tail=tail,
                                              sink_segments=sink_segments)
    return out
