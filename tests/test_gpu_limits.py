"""GPU parity at the library's size limits.

- Router and block-sparse attention at the largest block count (14,000 blocks of 64
  rows, ragged last block): the per-workgroup tile bitmaps are at full size and the
  router's score kernel falls back to one query block per workgroup (the scores of four
  no longer fit in LDS). Tile lists of sampled query blocks are compared bit for bit
  with the oracle's router steps, and their outputs with the oracle.
- Dense TARA with the largest key count of bf16 calls (2^23 keys, head_dim 128): the
  transposed V copy then spans just under 2^31 bytes per head, the edge of the 32-bit
  buffer range its loads use. Sampled query rows are compared with the oracle.

Both run on one head so that the oracle finishes in seconds."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_02_amd import api, workloads as W
from gpu_common import compare, f64, layout_device, to_device

pytestmark = pytest.mark.gpu


def test_router_and_sparse_at_block_limit():
    # 1,990 + 430,000 + 4,000 + 460,000 = 895,990 rows = 14,000 blocks (last one 54 rows);
    # video frames of 1,000 rows, so many tiles straddle two frames
    wl = W.custom("limit_blocks",
                  [W.Span(W.SEG_TEXT, 1990), W.Span(W.SEG_GUIDE, 430 * 1000, 430),
                   W.Span(W.SEG_AUDIO, 4000), W.Span(W.SEG_OUTPUT, 460 * 1000, 460)],
                  heads=1, head_dim=64, dtype="bf16", seed_index=80, frame_weight=0.7,
                  protected_prefix_len=1990)
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    plan = api.router_plan(seg, wl.protected_prefix_len, 0.9)
    nb, prot_ref, video, k_sel = oracle.router_plan(seg, wl.protected_prefix_len, 64, 0.9)
    assert nb == 14000 and plan["nb"] == nb and plan["k_sel"] == k_sel
    print(f"case {wl.name} n={wl.n} nb={nb} n_video={len(video)} k_sel={k_sel}", flush=True)
    tiles, prot = api.attn_block_router(qd, kd, seg_d, wl.protected_prefix_len, k_sel,
                                        plan["n_prot"])
    o, lse = api.attn_block_sparse(qd, kd, vd, seg_d, t_d, tiles, prot, *wl.tara,
                                   scale=wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(prot.cpu().numpy(), prot_ref)

    # the oracle's router steps for sampled query blocks
    rng = np.random.default_rng(80)
    blocks = sorted(set([0, 31, 32, 6750, 6751, 6781, 13999]) |
                    set(rng.integers(0, nb, 9).tolist()))
    qbar = oracle.block_means_fp32(W.to_float32(q[:, 0], "bf16"), 64)
    kbar = oracle.block_means_fp32(W.to_float32(k[:, 0], "bf16"), 64)
    ref_tiles = oracle.select_topk(oracle.pooled_scores_fp32(qbar[blocks], kbar[video]), video,
                                   k_sel)
    got_tiles = tiles[0].cpu().numpy()
    assert np.array_equal(got_tiles[blocks], ref_tiles)

    # the oracle attends over its own lists of the sampled blocks
    tl_ref = np.full((1, nb, k_sel), -1, dtype=np.int64)
    tl_ref[0, blocks] = ref_tiles
    ref = oracle.block_sparse(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), seg, t, wl.tara,
                              wl.scale, 64, prot_ref, tl_ref, heads=[0], qblocks=blocks)
    og, lg, orf, lrf = [], [], [], []
    for (_, qb), (ob, lb) in ref.items():
        lo, hi = qb * 64, min(wl.n, qb * 64 + 64)
        og.append(o[lo:hi, 0])
        lg.append(lse[lo:hi, 0])
        orf.append(ob)
        lrf.append(lb)
    compare(torch.cat(og), torch.cat(lg), np.concatenate(orf), np.concatenate(lrf), "bf16",
            "sparse at 14,000 blocks")


def test_dense_at_key_limit():
    # 8,608 + 4,000,000 + 380,000 + 4,000,000 = 8,388,608 = 2^23 key rows, head_dim 128
    wl = W.custom("limit_keys",
                  [W.Span(W.SEG_TEXT, 8608), W.Span(W.SEG_GUIDE, 4000 * 1000, 4000),
                   W.Span(W.SEG_AUDIO, 380000), W.Span(W.SEG_OUTPUT, 4000 * 1000, 4000)],
                  heads=1, head_dim=128, dtype="bf16", seed_index=81, frame_weight=0.7)
    assert wl.n == 1 << 23
    seg, t = W.layout(wl)
    q, k, v = W.make_qkv(wl)
    # 192 query rows of output video across the boundary of frames 999 and 1000
    a = 8608 + 4000000 + 380000 + 999 * 1000 + 904
    rows = slice(a, a + 192)
    kd, vd = to_device(k, "bf16"), to_device(v, "bf16")
    qd = to_device(np.ascontiguousarray(q[rows]), "bf16")
    seg_k, t_k = torch.from_numpy(seg).cuda(), torch.from_numpy(t).cuda()
    seg_q = torch.from_numpy(np.ascontiguousarray(seg[rows])).cuda()
    t_q = torch.from_numpy(np.ascontiguousarray(t[rows])).cuda()
    print(f"case {wl.name} nk={wl.n} nq=192 d=128", flush=True)
    o, lse = api.attn_dense_tara(qd, kd, vd, seg_q, t_q, seg_k, t_k, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    del kd, vd
    pick = [0, 95, 96, 191]
    o_ref, l_ref = oracle.dense_tara(f64(q[rows][pick], "bf16"), f64(k, "bf16"), f64(v, "bf16"),
                                     seg[rows][pick], t[rows][pick], seg, t, wl.tara, wl.scale)
    compare(o[pick], lse[pick], o_ref, l_ref, "bf16", "dense at 2^23 keys")
