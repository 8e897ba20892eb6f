"""Randomised GPU parity sweep.

Each case draws a packed layout (spans of text, guide video, audio and output video in
a random order, with random lengths and frame sizes, so tiles straddle frames and
segments and the last block is ragged), a head count, head_dim, dtype, TARA knobs and a
protected prefix, then checks against the float64 oracle:
- dense TARA and the partition path, every output row;
- the router (tile and protected lists bit-exact) and block-sparse attention at a random
  block size and sparsity, with or without the tail term and audio sink blocks, every
  output row;
- for bf16 at block sizes 64 and 128, the int8 QK product against the oracle's int8
  path.
A second set of cases takes the knobs to their extremes (protected prefixes 0 and n,
sparsity 0.99, strength up to 50 and cap up to 60, falloff 0.01, a second softmax scale)
and also feeds hand-built tile lists with repeated, negative and out-of-range entries.
A third set draws layouts with several guide-video spans and checks the reference-
protection router (Light / Heavy) and the attention over its lists.
The seeds are fixed, so every run draws the same cases."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_02_amd import api, workloads as W
from gpu_common import compare, f64, layout_device, to_device
from test_gpu_small import _route_oracle, _tails_oracle
from test_gpu_variants import _assemble

pytestmark = pytest.mark.gpu

KINDS = (W.SEG_TEXT, W.SEG_GUIDE, W.SEG_AUDIO, W.SEG_OUTPUT)


def _random_case(seed):
    rng = np.random.default_rng(9000 + seed)
    kinds = list(rng.permutation(KINDS)) + list(rng.choice(KINDS, size=int(rng.integers(0, 3))))
    spans = []
    for kind in kinds:
        if kind in (W.SEG_GUIDE, W.SEG_OUTPUT):
            frames = int(rng.integers(1, 7))
            spans.append(W.Span(int(kind), frames * int(rng.integers(1, 150)), frames))
        else:
            spans.append(W.Span(int(kind), int(rng.integers(1, 200))))
    n = sum(s.length for s in spans)
    dtype = str(rng.choice(["bf16", "f32"]))
    params = dict(strength=float(rng.choice([0.0, 0.5, 2.0, 7.0])),
                  window=float(rng.choice([0.0, 0.2, 0.5])),
                  falloff=float(rng.choice([0.1, 0.25, 1.0])),
                  cap=float(rng.choice([0.5, 6.0, 20.0])))
    wl = W.custom(f"random_{seed}", spans, heads=int(rng.integers(1, 4)),
                  head_dim=int(rng.choice([64, 128])), dtype=dtype, seed_index=200 + seed,
                  frame_weight=float(rng.choice([0.0, 0.7])),
                  protected_prefix_len=int(rng.integers(0, min(n, 300) + 1)), **params)
    sparse = dict(bs=int(rng.choice([32, 64, 128])), sparsity=float(rng.choice([0.0, 0.3, 0.8, 0.95])),
                  tail=bool(rng.integers(0, 2)), sinks=bool(rng.integers(0, 2)),
                  int8=bool(rng.integers(0, 2)))
    return wl, sparse


@pytest.mark.parametrize("seed", range(48))
def test_random_layouts(seed):
    wl, sp = _random_case(seed)
    dtype, H, d, bs = wl.dtype, wl.heads, wl.head_dim, sp["bs"]
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    q64, k64, v64 = f64(q, dtype), f64(k, dtype), f64(v, dtype)
    print(f"case {wl.name} n={wl.n} spans={[(s.seg, s.length, s.frames) for s in wl.spans]} "
          f"H={H} d={d} {dtype} tara={wl.tara} prefix={wl.protected_prefix_len} {sp}",
          flush=True)

    # dense and the partition path
    o_ref, l_ref = oracle.dense_tara(q64, k64, v64, seg, t, seg, t, wl.tara, wl.scale)
    o, lse = api.attn_dense_tara(qd, kd, vd, seg_d, t_d, seg_d, t_d, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, dtype, f"{wl.name} dense")
    o, lse = api.attn_dense_tara_via(qd, kd, vd, seg_d, t_d, seg, t, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, dtype, f"{wl.name} via")

    # router and block-sparse attention
    prefix = wl.protected_prefix_len
    plan = api.router_plan(seg, prefix, sp["sparsity"], block_size=bs)
    _, prot_ref, _, k_ref = oracle.router_plan(seg, prefix, bs, sp["sparsity"])
    assert plan["k_sel"] == k_ref and plan["n_prot"] == len(prot_ref)
    if sp["tail"]:
        tiles, prot, tl, tv = api.attn_block_router_tail(qd, kd, vd, seg_d, prefix, plan["k_sel"],
                                                         plan["n_prot"], scale=wl.scale,
                                                         block_size=bs)
    else:
        tiles, prot = api.attn_block_router(qd, kd, seg_d, prefix, plan["k_sel"],
                                            plan["n_prot"], block_size=bs)
        tl = tv = None
    sinks = (1 << W.SEG_AUDIO) if sp["sinks"] else 0
    o, lse = api.attn_block_sparse_sinks(qd, kd, vd, seg_d, t_d, tiles, prot, sinks, tl, tv,
                                         *wl.tara, scale=wl.scale, block_size=bs)
    torch.cuda.synchronize()
    tiles_ref = _route_oracle(wl, q, k, seg, plan["k_sel"], range(H), bs=bs)
    assert np.array_equal(prot.cpu().numpy(), prot_ref)
    assert np.array_equal(tiles.cpu().numpy(), tiles_ref)
    tails = _tails_oracle(wl, q, k, v, seg, tiles_ref, range(H), bs=bs) if sp["tail"] else None
    sink_segs = (W.SEG_AUDIO,) if sp["sinks"] else ()
    ref = oracle.block_sparse(q64, k64, v64, seg, t, wl.tara, wl.scale, bs, prot_ref, tiles_ref,
                              tails=tails, sink_segments=sink_segs)
    o_ref, l_ref = _assemble(ref, wl.n, H, d, bs)
    compare(o, lse, o_ref, l_ref, dtype, f"{wl.name} sparse")

    # int8 QK product (bf16 inputs, block sizes 64 and 128)
    if sp["int8"] and dtype == "bf16" and bs != 32:
        o, lse = api.attn_block_sparse_int8qk(qd, kd, vd, seg_d, t_d, tiles, prot, tail_lse=tl,
                                              tail_v=tv, sink_segments=sinks,
                                              strength=wl.strength, window=wl.window,
                                              falloff=wl.falloff, cap=wl.cap, scale=wl.scale,
                                              block_size=bs)
        torch.cuda.synchronize()
        ref = oracle.block_sparse(q64, k64, v64, seg, t, wl.tara, wl.scale, bs, prot_ref,
                                  tiles_ref, tails=tails, sink_segments=sink_segs, int8_qk=True)
        o_ref, l_ref = _assemble(ref, wl.n, H, d, bs)
        compare(o, lse, o_ref, l_ref, dtype, f"{wl.name} int8")


def _extreme_case(seed):
    rng = np.random.default_rng(7000 + seed)
    kinds = list(rng.permutation(KINDS)) + list(rng.choice(KINDS, size=int(rng.integers(0, 3))))
    spans = []
    for kind in kinds:
        if kind in (W.SEG_GUIDE, W.SEG_OUTPUT):
            frames = int(rng.integers(1, 9))
            spans.append(W.Span(int(kind), frames * int(rng.integers(1, 200)), frames))
        else:
            spans.append(W.Span(int(kind), int(rng.integers(1, 300))))
    n = sum(s.length for s in spans)
    prefix = int(rng.choice([0, n, int(rng.integers(0, n + 1))]))
    wl = W.custom(f"extreme_{seed}", spans, heads=int(rng.integers(1, 4)),
                  head_dim=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
                  seed_index=300 + seed, frame_weight=float(rng.choice([0.0, 0.7, 0.95])),
                  qk_gain=float(rng.choice([0.5, 1.0])), protected_prefix_len=prefix,
                  strength=float(rng.choice([0.0, 0.01, 50.0])),
                  window=float(rng.choice([0.0, 3.0])), falloff=float(rng.choice([0.01, 10.0])),
                  cap=float(rng.choice([0.0, 0.5, 60.0])))
    scale = float(rng.choice([wl.scale, 0.05]))
    return wl, scale, dict(bs=int(rng.choice([32, 64, 128])), sparsity=float(rng.choice([0.5, 0.99])),
                           tail=bool(rng.integers(0, 2)), sinks=bool(rng.integers(0, 2)),
                           hand=bool(rng.integers(0, 2))), rng


@pytest.mark.parametrize("seed", range(24))
def test_random_extremes(seed):
    """Protected prefixes 0 and n, sparsity 0.99, extreme TARA knobs (strength 0.01-50,
    cap 0-60, falloff 0.01-10, window 3 s), a second scale, and hand-built tile lists with
    repeats, -1 and out-of-range entries (a row with no key at all gives o = 0 and
    L = -inf on both sides)."""
    wl, scale, sp, rng = _extreme_case(seed)
    dtype, H, d, bs = wl.dtype, wl.heads, wl.head_dim, sp["bs"]
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    q64, k64, v64 = f64(q, dtype), f64(k, dtype), f64(v, dtype)
    print(f"case {wl.name} n={wl.n} H={H} d={d} {dtype} tara={wl.tara} scale={scale:.4g} "
          f"prefix={wl.protected_prefix_len} {sp}", flush=True)
    o_ref, l_ref = oracle.dense_tara(q64, k64, v64, seg, t, seg, t, wl.tara, scale)
    o, lse = api.attn_dense_tara(qd, kd, vd, seg_d, t_d, seg_d, t_d, *wl.tara, scale=scale)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, dtype, f"{wl.name} dense")

    prefix, nb = wl.protected_prefix_len, (wl.n + bs - 1) // bs
    tl = tv = tails = None
    if sp["hand"]:
        k_sel = int(rng.integers(1, 12))
        tiles_np = rng.integers(-2, nb + 3, size=(H, nb, k_sel)).astype(np.int32)
        prot_np = rng.integers(-1, nb + 2, size=int(rng.integers(0, 5))).astype(np.int32)
        tiles, prot = torch.from_numpy(tiles_np).cuda(), torch.from_numpy(prot_np).cuda()
    else:
        plan = api.router_plan(seg, prefix, sp["sparsity"], block_size=bs)
        if sp["tail"]:
            tiles, prot, tl, tv = api.attn_block_router_tail(qd, kd, vd, seg_d, prefix,
                                                             plan["k_sel"], plan["n_prot"],
                                                             scale=scale, block_size=bs)
        else:
            tiles, prot = api.attn_block_router(qd, kd, seg_d, prefix, plan["k_sel"],
                                                plan["n_prot"], block_size=bs)
        torch.cuda.synchronize()
        _, prot_np, _, _ = oracle.router_plan(seg, prefix, bs, sp["sparsity"])
        tiles_np = _route_oracle(wl, q, k, seg, plan["k_sel"], range(H), bs=bs)
        # the GPU lists must equal the oracle's; the oracle then runs on its own lists
        assert np.array_equal(prot.cpu().numpy(), prot_np)
        assert np.array_equal(tiles.cpu().numpy(), tiles_np)
        if sp["tail"]:
            tails = {h: oracle.tail_terms(W.to_float32(q[:, h], dtype), W.to_float32(k[:, h], dtype),
                                          v64[:, h], seg, prefix, bs, tiles_np[h], scale)
                     for h in range(H)}
    sinks = (1 << W.SEG_AUDIO) if sp["sinks"] else 0
    o, lse = api.attn_block_sparse_sinks(qd, kd, vd, seg_d, t_d, tiles, prot, sinks, tl, tv,
                                         *wl.tara, scale=scale, block_size=bs)
    torch.cuda.synchronize()
    ref = oracle.block_sparse(q64, k64, v64, seg, t, wl.tara, scale, bs, prot_np, tiles_np,
                              tails=tails, sink_segments=(W.SEG_AUDIO,) if sp["sinks"] else ())
    o_ref, l_ref = _assemble(ref, wl.n, H, d, bs)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse.cpu().numpy()), empty)
    if empty.any():
        assert np.all(o.float().cpu().numpy()[empty] == 0)
        l_ref = np.where(empty, 0.0, l_ref)
        lse = torch.where(torch.isneginf(lse), torch.zeros_like(lse), lse)
    compare(o, lse, o_ref, l_ref, dtype, f"{wl.name} sparse")


def _reference_case(seed):
    """A packed layout with one to three guide-video spans apart from each other (each one
    or more reference ranges), a protected prefix, and a random reference mode."""
    rng = np.random.default_rng(11000 + seed)
    n_guides = int(rng.integers(1, 4))
    spans = [W.Span(W.SEG_TEXT, int(rng.integers(1, 150)))]
    for g in range(n_guides):
        frames = int(rng.integers(1, 6))
        spans.append(W.Span(W.SEG_GUIDE, frames * int(rng.integers(20, 220)), frames))
        spans.append(W.Span(int(rng.choice([W.SEG_AUDIO, W.SEG_OUTPUT, W.SEG_TEXT])),
                            int(rng.integers(1, 300))))
    frames = int(rng.integers(1, 6))
    spans.append(W.Span(W.SEG_OUTPUT, frames * int(rng.integers(40, 300)), frames))
    wl = W.custom(f"reference_{seed}", spans, heads=int(rng.integers(1, 4)),
                  head_dim=int(rng.choice([64, 128])), dtype="bf16", seed_index=500 + seed,
                  frame_weight=float(rng.choice([0.0, 0.7])),
                  protected_prefix_len=int(rng.integers(0, spans[0].length + 1)))
    return wl, dict(bs=int(rng.choice([32, 64, 128])),
                    sparsity=float(rng.choice([0.0, 0.5, 0.85, 0.95])),
                    mode=int(rng.choice([api.H3_REF_LIGHT, api.H3_REF_HEAVY])))


@pytest.mark.parametrize("seed", range(16))
def test_random_reference_protection(seed):
    """Reference protection ("H3 SLA Attention", inputs table) on random layouts with
    several guide spans: the quota router's lists and protected list bit-exact against the
    oracle, then block-sparse attention over the oracle's lists, every output row."""
    from gpu_common import checked_routes_ref
    from oracle.router import REF_HEAVY, REF_LIGHT
    wl, sp = _reference_case(seed)
    H, d, bs = wl.heads, wl.head_dim, sp["bs"]
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    print(f"case {wl.name} n={wl.n} spans={[(s.seg, s.length, s.frames) for s in wl.spans]} "
          f"H={H} d={d} prefix={wl.protected_prefix_len} {sp}", flush=True)
    tiles, prot = api.attn_block_router_ref(qd, kd, seg_d, seg, wl.protected_prefix_len,
                                            sp["sparsity"], sp["mode"], block_size=bs)
    torch.cuda.synchronize()
    mode = REF_LIGHT if sp["mode"] == api.H3_REF_LIGHT else REF_HEAVY
    tiles_ref, prot_ref = checked_routes_ref(tiles, prot, wl, q, k, seg, sp["sparsity"], mode,
                                             range(H), bs=bs, tag=wl.name)
    o, lse = api.attn_block_sparse(qd, kd, vd, seg_d, t_d, tiles if tiles.shape[-1] else None,
                                   prot if prot.numel() else None, *wl.tara, scale=wl.scale,
                                   block_size=bs)
    torch.cuda.synchronize()
    ref = oracle.block_sparse(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), seg, t, wl.tara,
                              wl.scale, bs, prot_ref, tiles_ref)
    o_ref, l_ref = _assemble(ref, wl.n, H, d, bs)
    compare(o, lse, o_ref, l_ref, "bf16", f"{wl.name} reference sparse")
