"""Dense TARA attention, plain attention, the stable LSE merge and the
positive-partition decomposition, in float64 (test infrastructure only).

Sources (web pages):
- "Flash Partitions for H3 native temporal alignment", section 1 ("What
  receives the temporal bias?"): the penalty, its edge selection and the
  modified score.
- same page, section 3 ("Decompose the same rule into positive
  contributions"): the split exp(-p) = exp(-cap) + [exp(-p) - exp(-cap)] into
  three contribution kinds, and the correction threshold.
- same page, section 4 ("Why log-sum-exp is necessary"): the LSE merge,
  zero-weight omission, expm1 weights, output-frame chunks, the off-switch.
- "TARA : alignement temporel natif pour les références MiniMax H3", section
  "La règle temporelle": the same rule and defaults restated.
"""
from __future__ import annotations

import math

import numpy as np

SEG_TEXT, SEG_GUIDE, SEG_AUDIO, SEG_OUTPUT = 0, 1, 2, 3


def tara_penalty(dt, strength, window, falloff, cap):
    """penalty(dt) = min(strength * (max(dt - window, 0) / falloff)^2, cap).

    Flash Partitions page, section 1. ``dt`` is an absolute time difference
    in seconds (scalar or array); computed in float64.
    """
    dt = np.asarray(dt, dtype=np.float64)
    x = np.maximum(dt - window, 0.0) / falloff
    return np.minimum(strength * (x * x), cap)


def tara_bias(seg_q, t_q, seg_k, t_k, params):
    """Penalty matrix [len(q rows), len(k rows)] subtracted from the scores.

    Only pairs (output-video query, guide-video key) are affected; every other
    edge keeps the ordinary rule (Flash Partitions page, section 1). The
    timestamps are the float32 row times, widened to float64.
    """
    strength, window, falloff, cap = params
    seg_q = np.asarray(seg_q)
    seg_k = np.asarray(seg_k)
    tq = np.asarray(t_q, dtype=np.float32).astype(np.float64)
    tk = np.asarray(t_k, dtype=np.float32).astype(np.float64)
    affected = (seg_q[:, None] == SEG_OUTPUT) & (seg_k[None, :] == SEG_GUIDE)
    dt = np.abs(tq[:, None] - tk[None, :])
    pen = tara_penalty(dt, strength, window, falloff, cap)
    return np.where(affected, pen, 0.0)


def _softmax_rows(s, v):
    """Softmax over the last axis of scores ``s`` (float64) applied to ``v``.

    Returns (o, lse) with lse the natural-log normaliser, computed with the
    row maximum subtracted first.
    """
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    o = (e @ v) / den
    lse = (m + np.log(den))[:, 0]
    return o, lse


def dense_tara(q, k, v, seg_q, t_q, seg_k, t_k, params, scale, row_chunk=256):
    """Dense attention with the TARA penalty, exact float64.

    q: [nq, H, d]; k, v: [nk, H, d] (float64 views of the stored inputs).
    For each head h and query row i:
        s_ij = scale * (q_i . k_j) - p_ij,
        p_ij = penalty(|t_i - t_j|) if seg_i is output video and seg_j is guide
               video, else 0,
        L_i  = ln sum_j exp(s_ij),   o_i = sum_j exp(s_ij - L_i) v_j.
    Returns o [nq, H, d] and lse [nq, H] (natural log), both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, H, d = q.shape
    o = np.empty((nq, H, d))
    lse = np.empty((nq, H))
    kh = [np.ascontiguousarray(k[:, h, :]) for h in range(H)]
    vh = [np.ascontiguousarray(v[:, h, :]) for h in range(H)]
    for r0 in range(0, nq, row_chunk):
        r1 = min(nq, r0 + row_chunk)
        pen = tara_bias(seg_q[r0:r1], t_q[r0:r1], seg_k, t_k, params)
        for h in range(H):
            s = scale * (q[r0:r1, h, :] @ kh[h].T) - pen
            o[r0:r1, h, :], lse[r0:r1, h] = _softmax_rows(s, vh[h])
    return o, lse


def plain_attention(q, k, v, scale):
    """Ordinary softmax attention (no penalty) of q [nq,H,d] over k, v [nk,H,d].

    This is one partition call of the Flash Partitions backend: a normalised
    local result together with its natural-log normaliser (section 4).
    """
    nq, H, d = q.shape
    o = np.empty((nq, H, d))
    lse = np.empty((nq, H))
    for h in range(H):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        o[:, h, :], lse[:, h] = _softmax_rows(s, v[:, h, :])
    return o, lse


def lse_merge(parts):
    """Merge partition results (o_i, lse_i, log_w_i) into (o, lse).

    Flash Partitions page, section 4:
        adjusted_L_i = L_i + log(w_i),
        L = logsumexp(adjusted_L_1, adjusted_L_2, ...),
        O = sum_i exp(adjusted_L_i - L) * O_i.
    o_i: [rows, H, d]; lse_i: [rows, H]; log_w_i: scalar or [rows, H].
    Rows where every adjusted normaliser is -inf get O = 0 and L = -inf.
    """
    adj = [np.asarray(l, dtype=np.float64) + np.asarray(w, dtype=np.float64)
           for (_, l, w) in parts]
    adj = np.stack(np.broadcast_arrays(*adj))          # [P, rows, H]
    m = adj.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    tot = np.exp(adj - m_safe[None]).sum(axis=0)
    L = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    L_safe = np.where(finite, L, 0.0)
    o = np.zeros(parts[0][0].shape)
    for (oi, _, _), a in zip(parts, adj):
        wgt = np.where(finite, np.exp(a - L_safe), 0.0)
        o = o + wgt[..., None] * np.asarray(oi, dtype=np.float64)
    return o, L


def runs(mask):
    """Maximal contiguous runs [start, end) where ``mask`` is true."""
    mask = np.asarray(mask, dtype=bool)
    out = []
    i, n = 0, len(mask)
    while i < n:
        if mask[i]:
            j = i
            while j < n and mask[j]:
                j += 1
            out.append((i, j))
            i = j
        else:
            i += 1
    return out


def _frames(seg, t, kind):
    """Video frames of segment ``kind``: runs of rows with equal timestamp."""
    out = []
    for a, b in runs(np.asarray(seg) == kind):
        s = a
        for r in range(a + 1, b + 1):
            if r == b or t[r] != t[s]:
                out.append((s, r, float(np.float32(t[s]))))
                s = r
    return out


def tara_partitions(q, k, v, seg, t, params, scale, frame_chunk=8):
    """The same result as ``dense_tara`` (self-attention over one packed
    sequence) computed by the positive-contribution decomposition.

    Flash Partitions page, sections 3 and 4. Because 0 <= penalty <= cap,
    exp(-p) = exp(-cap) + [exp(-p) - exp(-cap)] with both terms nonnegative,
    so for the queries of an output frame f the key set splits into:
      - every non-guide key run, multiplier 1;
      - every guide key run, uniform multiplier exp(-cap);
      - the keys of each guide frame g, multiplier exp(-p(|t_f - t_g|)) -
        exp(-cap), written exp(-cap) * expm1(cap - p) and omitted when zero.
    Each part is an ordinary attention call returning (O_i, L_i); the parts are
    merged with ``lse_merge``. Queries outside the output video get one
    ordinary full attention call. Output frames are processed in chunks of
    ``frame_chunk`` frames; the chunk size bounds buffers and must not change
    the result.
    """
    strength, window, falloff, cap = params
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    seg = np.asarray(seg)
    t = np.asarray(t, dtype=np.float32)
    n, H, d = q.shape
    o = np.empty((n, H, d))
    lse = np.empty((n, H))

    # Queries outside the output video: one ordinary call over every key.
    for a, b in runs(seg != SEG_OUTPUT):
        o[a:b], lse[a:b] = plain_attention(q[a:b], k, v, scale)

    nonguide_runs = runs(seg != SEG_GUIDE)
    guide_runs = runs(seg == SEG_GUIDE)
    guide_frames = _frames(seg, t, SEG_GUIDE)
    out_frames = _frames(seg, t, SEG_OUTPUT)
    base = -float(cap)                      # log of the uniform multiplier exp(-cap)

    for c0 in range(0, len(out_frames), frame_chunk):
        chunk = out_frames[c0:c0 + frame_chunk]
        rows = np.concatenate([np.arange(a, b) for a, b, _ in chunk])
        qc = q[rows]
        parts = []
        for a, b in nonguide_runs:
            oi, li = plain_attention(qc, k[a:b], v[a:b], scale)
            parts.append((oi, li, 0.0))
        for a, b in guide_runs:
            oi, li = plain_attention(qc, k[a:b], v[a:b], scale)
            parts.append((oi, li, base))
        # Local corrections: one part per (output frame, guide frame) pair,
        # covering only that output frame's rows within the chunk.
        offs = 0
        for fa, fb, tf in chunk:
            nr = fb - fa
            for ga, gb, tg in guide_frames:
                pen = float(tara_penalty(abs(np.float64(tf) - np.float64(tg)),
                                         strength, window, falloff, cap))
                corr = math.expm1(cap - pen)   # exp(-p) - exp(-cap) = exp(-cap) * expm1(cap - p)
                if corr <= 0.0:
                    continue                   # zero-weight correction: omitted
                oi_f, li_f = plain_attention(q[fa:fb], k[ga:gb], v[ga:gb], scale)
                oi = np.zeros((len(rows), H, d))
                li = np.full((len(rows), H), -np.inf)
                oi[offs:offs + nr] = oi_f
                li[offs:offs + nr] = li_f
                parts.append((oi, li, base + math.log(corr)))
            offs += nr
        o[rows], lse[rows] = lse_merge(parts)
    return o, lse
