"""Seeded synthetic inputs for the packed-sequence attention workloads.

This module holds layouts, seeds and value recipes only. It computes no
attention, no penalty, no pooling and no routing, so the CPU oracle tests and
the GPU path can both draw their inputs from it without sharing any of the
method's arithmetic.

Packed sequence (H3 Flash Partitions page, section 1): text, guide (motion
reference) video, audio and output video rows share one self-attention call.
Every row carries a segment id and a timestamp in seconds. Video latent frame
``k`` is stamped ``float32(k / 6)`` (24 fps with a four-frame latent stride);
text and audio rows carry 0.

Value recipe, per workload ``c``: ``numpy.random.SeedSequence(1000 + c)`` is
spawned into ``4 * heads`` independent streams, one per (tensor, head) with
tensor in (q, k, v, frame component). Values are float64 standard normals,
combined per the recipe, rounded to float32 (round to nearest even) and, for
bf16 workloads, to bf16 (round to nearest even). Both sides read the same bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Iterable, Sequence

import numpy as np

SEG_TEXT = 0     # text tokens, including text padding
SEG_GUIDE = 1    # guide (motion reference) video latents
SEG_AUDIO = 2    # audio rows (80 rows per second)
SEG_OUTPUT = 3   # output (generated) video latents

FRAME_SECONDS = 1.0 / 6.0  # 24 fps, one latent frame per 4 video frames

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_FRAME = 0, 1, 2, 3


@dataclass(frozen=True)
class Span:
    """A contiguous run of rows of one segment kind.

    ``frames`` > 0 marks a video span of ``frames`` latent frames of
    ``length // frames`` rows each.
    """
    seg: int
    length: int
    frames: int = 0


@dataclass(frozen=True)
class Workload:
    name: str
    spans: tuple
    heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    seed_index: int
    qk_gain: float = 1.0       # multiplies the q and k draws (0.5 in the 6,800-row case)
    frame_weight: float = 0.0  # weight of the per-frame shared q/k component
    strength: float = 2.0
    window: float = 0.20
    falloff: float = 0.25
    cap: float = 6.0
    block_size: int = 64
    sparsities: tuple = ()
    protected_prefix_len: int = 0
    description: str = ""

    @property
    def n(self) -> int:
        return sum(s.length for s in self.spans)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def tara(self) -> tuple:
        return (self.strength, self.window, self.falloff, self.cap)


def _video(seg: int, frames: int, per_frame: int) -> Span:
    return Span(seg, frames * per_frame, frames)


# 304 rows: 16 text, guide 8 x 16, 32 audio, output 8 x 16. fp32, 1 head, d 64.
TINY_DENSE = Workload(
    name="tiny_dense_tara_304x1_d64_f32",
    spans=(Span(SEG_TEXT, 16), _video(SEG_GUIDE, 8, 16), Span(SEG_AUDIO, 32),
           _video(SEG_OUTPUT, 8, 16)),
    heads=1, head_dim=64, dtype="f32", seed_index=1,
    description="tiny dense TARA, fp32")

# 6,800 rows: 256 text, guide 12 x 256, 400 audio, output 12 x 256. bf16, 24 heads.
MID_DENSE = Workload(
    name="dense_tara_6800x24_d128_bf16",
    spans=(Span(SEG_TEXT, 256), _video(SEG_GUIDE, 12, 256), Span(SEG_AUDIO, 400),
           _video(SEG_OUTPUT, 12, 256)),
    heads=24, head_dim=128, dtype="bf16", seed_index=2, qk_gain=0.5,
    description="dense TARA, bf16")

# 31,552 rows (493 blocks of 64): 512 text + 40 padding, 400 audio, guide
# 15 x 1,020, output 15 x 1,020. Protected prefix = the first 952 rows.
MID_SPARSE = Workload(
    name="block_sparse_31552x24_d128_bf16",
    spans=(Span(SEG_TEXT, 552), Span(SEG_AUDIO, 400), _video(SEG_GUIDE, 15, 1020),
           _video(SEG_OUTPUT, 15, 1020)),
    heads=24, head_dim=128, dtype="bf16", seed_index=3, frame_weight=0.7,
    strength=0.0, sparsities=(0.85,), protected_prefix_len=952,
    description="block-sparse, bf16, no penalty")

# 116,883 rows: 512 text + 6,747 padding, guide 31 x 1,752, 1,000 audio,
# output 31 x 1,752. The per-frame shared component uses the same seed as the
# sparse sweep so that the dense and sparse calls see identical inputs.
FULL_DENSE = Workload(
    name="dense_tara_116883x56_d128_bf16",
    spans=(Span(SEG_TEXT, 7259), _video(SEG_GUIDE, 31, 1752), Span(SEG_AUDIO, 1000),
           _video(SEG_OUTPUT, 31, 1752)),
    heads=56, head_dim=128, dtype="bf16", seed_index=5, frame_weight=0.7,
    protected_prefix_len=7259,
    description="full-scale dense TARA, bf16")

FULL_SPARSE = Workload(
    name="block_sparse_tara_116883x56_d128_bf16",
    spans=FULL_DENSE.spans,
    heads=56, head_dim=128, dtype="bf16", seed_index=5, frame_weight=0.7,
    sparsities=(0.50, 0.70, 0.85, 0.90, 0.95), protected_prefix_len=7259,
    description="full-scale block-sparse with TARA on routed guide tiles, bf16")

# The isolated attention shape timed on the Flash Partitions page (section 5): 107,126
# tokens, 8 heads, d 128, bf16. The page gives no segment layout; this one keeps the
# full-scale proportions: 5,126 text, guide 28 x 1,800, 1,200 audio, output 28 x 1,800.
P1_MICRO = Workload(
    name="dense_tara_107126x8_d128_bf16",
    spans=(Span(SEG_TEXT, 5126), _video(SEG_GUIDE, 28, 1800), Span(SEG_AUDIO, 1200),
           _video(SEG_OUTPUT, 28, 1800)),
    heads=8, head_dim=128, dtype="bf16", seed_index=6, frame_weight=0.7,
    protected_prefix_len=5126,
    description="isolated dense TARA shape of the Flash Partitions page, bf16")

WORKLOADS = {w.name: w for w in (TINY_DENSE, MID_DENSE, MID_SPARSE, FULL_DENSE, FULL_SPARSE,
                                 P1_MICRO)}


def layout(w: Workload):
    """Per-row segment ids (uint8) and timestamps (float32 seconds)."""
    seg = np.empty(w.n, dtype=np.uint8)
    t = np.zeros(w.n, dtype=np.float32)
    r = 0
    for s in w.spans:
        seg[r:r + s.length] = s.seg
        if s.frames:
            per = s.length // s.frames
            for f in range(s.frames):
                t[r + f * per:r + (f + 1) * per] = np.float32(f / 6.0)
        r += s.length
    return seg, t


def frame_ids(w: Workload) -> np.ndarray:
    """Index of each row's video frame across all video spans (-1 outside video)."""
    fid = np.full(w.n, -1, dtype=np.int64)
    r = 0
    nf = 0
    for s in w.spans:
        if s.frames:
            per = s.length // s.frames
            for f in range(s.frames):
                fid[r + f * per:r + (f + 1) * per] = nf
                nf += 1
        r += s.length
    return fid


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(w: Workload):
    return np.random.SeedSequence(1000 + w.seed_index).spawn(4 * w.heads)


def _video_frames(w: Workload):
    """(first row, last row + 1, global frame index) of every video frame."""
    out = []
    r = 0
    nf = 0
    for s in w.spans:
        if s.frames:
            per = s.length // s.frames
            for f in range(s.frames):
                out.append((r + f * per, r + (f + 1) * per, nf))
                nf += 1
        r += s.length
    return out


def _head_values(w: Workload, children, tensor: int, h: int, frames) -> np.ndarray:
    """float64 [n, d] values of one tensor for one head, before rounding."""
    rng = np.random.Generator(np.random.PCG64(children[tensor * w.heads + h]))
    z = rng.standard_normal((w.n, w.head_dim))
    if tensor == TENSOR_V:
        return z
    if w.frame_weight > 0.0 and frames:
        frng = np.random.Generator(np.random.PCG64(children[TENSOR_FRAME * w.heads + h]))
        c = frng.standard_normal((len(frames), w.head_dim))
        a = w.frame_weight
        b = float(np.sqrt(1.0 - a * a))
        for r0, r1, f in frames:
            z[r0:r1] = a * c[f] + b * z[r0:r1]
    if w.qk_gain != 1.0:
        z = w.qk_gain * z
    return z


def make_qkv(w: Workload, heads: Sequence[int] | None = None, workers: int | None = None):
    """Seeded q, k, v of shape [n, len(heads), d].

    fp32 workloads return float32 arrays; bf16 workloads return uint16 bf16
    bit patterns. ``heads`` selects a subset (the values of head ``h`` do not
    depend on which other heads are drawn). Streams are drawn in parallel
    threads; every stream is independent, so the values do not depend on the
    thread count.
    """
    hs = list(range(w.heads)) if heads is None else list(heads)
    children = _streams(w)
    frames = _video_frames(w)
    out_dtype = np.float32 if w.dtype == "f32" else np.uint16
    out = [np.empty((w.n, len(hs), w.head_dim), dtype=out_dtype) for _ in range(3)]

    def fill(job):
        tensor, j = job
        x32 = _head_values(w, children, tensor, hs[j], frames).astype(np.float32)
        out[tensor][:, j, :] = x32 if w.dtype == "f32" else f32_to_bf16_bits(x32)

    jobs = [(tensor, j) for tensor in (TENSOR_Q, TENSOR_K, TENSOR_V) for j in range(len(hs))]
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if workers <= 1 or len(jobs) == 1:
        for job in jobs:
            fill(job)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, jobs))
    return tuple(out)


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored input values (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def to_float32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of stored input values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def custom(name: str, spans: Iterable[Span], heads: int, head_dim: int, dtype: str,
           seed_index: int, **kw) -> Workload:
    """A workload with an arbitrary layout (used for ragged and edge cases)."""
    return Workload(name=name, spans=tuple(spans), heads=heads, head_dim=head_dim,
                    dtype=dtype, seed_index=seed_index, **kw)
