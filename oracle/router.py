"""Pooled block routing for block-sparse attention (test infrastructure only).

Sources (web pages):
- "H3 SLA Attention" node page, "How it works": one small product of block-mean
  queries with block-mean keys rates every (query block, key block) pair, and a
  query block attends only its best-rated (1 - sparsity_ratio) share of key
  blocks; no weights are learned, the choice comes from Q and K at run time.
- same page, "The inputs that matter" and the inputs table: sparsity_ratio is
  the fraction of key blocks skipped and 0.0 disables sparsity; block_size 64;
  with protect_audio, the blocks that hold language tokens or audio segments (the
  [text | cond | audio] part of the sequence) are attended by every query block.
- "H3 sparse-attention breakpoints" page: the density is a fraction of the
  video key/value tiles, while the text and audio context stays whole.

Readings where the pages are silent (each listed in the design notes):
- pooled vector = mean of the block's valid rows, accumulated in float32 in
  row order from +0.0, then divided by the row count (correctly rounded);
- pooled score = sum over d = 0..D-1 of fl32(qbar[d] * kbar[d]), each product
  rounded to float32 and added in order, no fused multiply-add, unscaled;
- k = min(n_video, max(1, ceil((1 - s) * n_video - 1e-9))) in float64, and
  k = n_video at s = 0;
- ranking: higher score first, ties to the lower tile index, NaN last; the
  chosen tiles are reported in ascending tile order;
- every query block is routed (text and audio query blocks included), each
  head separately.

Reference protection ("H3 SLA Attention", inputs table, reference_protection; the guide
video is the visual reference of the packed sequence):
- Off: no quota; reference tiles compete in the ordinary top-k.
- Heavy: every video tile that holds a guide row is protected (attended by every query
  block); the ordinary top-k runs over the remaining video tiles.
- Light: the ordinary top-k over all video tiles, and in addition, for each reference
  range (a maximal run of video tiles with consecutive block indices that hold a guide
  row), the best-scoring tiles of that range at a fixed reference sparsity of 0.85, i.e.
  select_count(n_range, 0.85) tiles. A query block attends the union; sparsity 0 still
  routes every tile.
"""
from __future__ import annotations

import math

import numpy as np

SEG_TEXT, SEG_GUIDE, SEG_AUDIO, SEG_OUTPUT = 0, 1, 2, 3


def select_count(n_video, sparsity):
    """Number of routed video tiles per query block (top 1 - sparsity)."""
    if n_video <= 0:
        return 0
    if sparsity == 0.0:
        return n_video
    k = math.ceil((1.0 - float(sparsity)) * n_video - 1e-9)
    return min(n_video, max(1, k))


def router_plan(seg, protected_prefix_len, block_size, sparsity):
    """Protected and video tiles of a packed sequence, and the routed count.

    A key block is protected when it overlaps rows [0, protected_prefix_len)
    or holds any text or audio row; all other blocks are video tiles.
    Returns (nb, protected block indices, video block indices, k).
    """
    seg = np.asarray(seg)
    n = len(seg)
    nb = (n + block_size - 1) // block_size
    protected = []
    video = []
    for b in range(nb):
        lo, hi = b * block_size, min(n, (b + 1) * block_size)
        rows = seg[lo:hi]
        if lo < protected_prefix_len or np.any((rows == SEG_TEXT) | (rows == SEG_AUDIO)):
            protected.append(b)
        else:
            video.append(b)
    prot = np.array(protected, dtype=np.int64)
    vid = np.array(video, dtype=np.int64)
    return nb, prot, vid, select_count(len(vid), sparsity)


def block_means_fp32(x32, block_size):
    """Per-block mean of float32 rows x32 [n, d] -> [nb, d] float32.

    Rows are added one at a time in row order starting from +0.0 (every
    addition rounded to float32), then the sum is divided by the number of
    valid rows in the block.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    n, d = x32.shape
    nb = (n + block_size - 1) // block_size
    out = np.empty((nb, d), dtype=np.float32)
    nfull = n // block_size
    if nfull:
        xb = x32[:nfull * block_size].reshape(nfull, block_size, d)
        acc = np.zeros((nfull, d), dtype=np.float32)
        for j in range(block_size):
            acc = acc + xb[:, j, :]
        out[:nfull] = acc / np.float32(block_size)
    if nb > nfull:
        acc = np.zeros(d, dtype=np.float32)
        for r in range(nfull * block_size, n):
            acc = acc + x32[r]
        out[nfull] = acc / np.float32(n - nfull * block_size)
    return out


def pooled_scores_fp32(qbar, kbar):
    """Pooled score matrix [nq_blocks, nk_tiles] float32 from qbar [nqb, d] and
    kbar [nkt, d]: sum over d in order of float32-rounded products."""
    qbar = np.asarray(qbar, dtype=np.float32)
    kbar = np.asarray(kbar, dtype=np.float32)
    s = np.zeros((qbar.shape[0], kbar.shape[0]), dtype=np.float32)
    for j in range(qbar.shape[1]):
        s = s + np.multiply.outer(qbar[:, j], kbar[:, j])
    return s


def select_topk(scores, video, k):
    """Top-k video tiles per row of ``scores`` [nqb, n_video] -> [nqb, k] int64.

    Higher score first; equal scores go to the lower tile index; NaN ranks
    after every number. The chosen global block indices are returned in
    ascending order.
    """
    scores = np.asarray(scores, dtype=np.float32)
    nqb, nv = scores.shape
    if k == 0:
        return np.zeros((nqb, 0), dtype=np.int64)
    idx = np.broadcast_to(np.arange(nv), (nqb, nv))
    neg = -scores.astype(np.float64)           # NaN stays NaN and sorts last
    order = np.lexsort((idx, neg), axis=-1)
    chosen = np.asarray(video)[order[:, :k]]
    return np.sort(chosen, axis=1)


def route_head(q32_h, k32_h, seg, protected_prefix_len, block_size, k):
    """Routing of one head: tile lists [nqb, k] (ascending block indices).

    q32_h, k32_h: [n, d] float32 (exact input values).
    """
    _, _, video, _ = router_plan(seg, protected_prefix_len, block_size, 0.0)
    qbar = block_means_fp32(q32_h, block_size)
    kbar = block_means_fp32(k32_h, block_size)
    scores = pooled_scores_fp32(qbar, kbar[video])
    return select_topk(scores, video, k)


REF_OFF, REF_LIGHT, REF_HEAVY = 0, 1, 2
LIGHT_REFERENCE_SPARSITY = 0.85


def reference_ranges(seg, protected_prefix_len, block_size):
    """Video tiles that hold a guide (visual reference) row, as ranges of consecutive
    block indices: a list of arrays of block indices, in ascending order."""
    seg = np.asarray(seg)
    n = len(seg)
    _, _, video, _ = router_plan(seg, protected_prefix_len, block_size, 0.0)
    ref = [int(b) for b in video
           if np.any(seg[b * block_size:min(n, (b + 1) * block_size)] == SEG_GUIDE)]
    ranges = []
    for b in ref:
        if ranges and ranges[-1][-1] == b - 1:
            ranges[-1].append(b)
        else:
            ranges.append([b])
    return [np.array(r, dtype=np.int64) for r in ranges]


def router_plan_ref(seg, protected_prefix_len, block_size, sparsity, mode):
    """Routing plan under a reference-protection mode.

    Returns (nb, protected blocks, routed-candidate video tiles, k, quotas): k is the
    ordinary top-k count over the candidates, and quotas a list of (range tiles, count)
    guaranteed per reference range (Light only). The tile-list width a query block
    needs is k + the sum of the quota counts, at most the number of candidates.
    """
    nb, prot, video, k = router_plan(seg, protected_prefix_len, block_size, sparsity)
    if mode == REF_OFF:
        return nb, prot, video, k, []
    ranges = reference_ranges(seg, protected_prefix_len, block_size)
    if mode == REF_HEAVY:
        ref = set(int(b) for r in ranges for b in r)
        prot = np.array(sorted(set(prot.tolist()) | ref), dtype=np.int64)
        video = np.array([b for b in video if int(b) not in ref], dtype=np.int64)
        return nb, prot, video, select_count(len(video), sparsity), []
    if mode == REF_LIGHT:
        quotas = [(r, select_count(len(r), LIGHT_REFERENCE_SPARSITY)) for r in ranges]
        return nb, prot, video, k, quotas
    raise ValueError(f"unknown reference-protection mode {mode}")


def route_head_ref(q32_h, k32_h, seg, protected_prefix_len, block_size, sparsity, mode):
    """Routing of one head under a reference-protection mode: per query block, the
    ascending union of the ordinary top-k over the candidate video tiles and (Light)
    each reference range's quota of its best-scoring tiles, padded with -1 to the
    list width min(k + sum of quotas, candidates). Returns [nqb, width] int64."""
    nb, _, video, k, quotas = router_plan_ref(seg, protected_prefix_len, block_size,
                                              sparsity, mode)
    width = min(k + sum(c for _, c in quotas), len(video))
    qbar = block_means_fp32(q32_h, block_size)
    kbar = block_means_fp32(k32_h, block_size)
    chosen = [set() for _ in range(nb)]
    parts = [(video, k)] + list(quotas)
    for tiles, count in parts:
        if count == 0 or len(tiles) == 0:
            continue
        picked = select_topk(pooled_scores_fp32(qbar, kbar[tiles]), tiles, count)
        for qb in range(nb):
            chosen[qb].update(int(b) for b in picked[qb])
    out = np.full((nb, width), -1, dtype=np.int64)
    for qb in range(nb):
        row = sorted(chosen[qb])
        out[qb, :len(row)] = row
    return out
