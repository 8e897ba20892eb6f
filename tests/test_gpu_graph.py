"""HIP graph capture of the hot path.

Every entry point takes caller-owned buffers and a stream, allocates nothing and never
waits on the host, so a caller can capture a whole step into one graph: here the dense
TARA call, the partition ("via") path with its merges, the router with the tail terms,
block-sparse attention with the tail term and the int8 QK product. The graph is replayed
several times, with eager work (the outputs cleared) and synchronizations between the
replays, and every replay must reproduce the eager results bit for bit: each kernel is
deterministic (fixed reduction orders; the only atomics are order-independent ORs into
tile bitmaps)."""
import pytest
import torch

from block_sparse_attention_02_amd import api, workloads as W
from gpu_common import layout_device, to_device

pytestmark = pytest.mark.gpu


def _workload():
    # frames of 37 and 45 rows: tiles straddle frames and segments; n not a multiple of 64
    return W.custom("graph_ragged",
                    [W.Span(W.SEG_TEXT, 29), W.Span(W.SEG_GUIDE, 9 * 37, 9),
                     W.Span(W.SEG_AUDIO, 51), W.Span(W.SEG_OUTPUT, 9 * 45, 9),
                     W.Span(W.SEG_TEXT, 13)],
                    heads=3, head_dim=128, dtype="bf16", seed_index=71, frame_weight=0.5)


def test_graph_replays_match_eager():
    wl = _workload()
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    n, H, D = qd.shape
    nb = (n + 63) // 64
    dev = qd.device
    plan = api.router_plan(seg, wl.protected_prefix_len, 0.6)  # host only: before capture
    k_sel, n_prot = plan["k_sel"], plan["n_prot"]
    print(f"case {wl.name} n={n} H={H} d={D} k_sel={k_sel} n_prot={n_prot}", flush=True)

    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)

    def ws(nbytes):
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)

    o_dense, o_via, o_sp, o_q8 = (torch.empty_like(qd) for _ in range(4))
    l_dense, l_via, l_sp, l_q8 = (torch.empty((n, H), **f32) for _ in range(4))
    tiles = torch.empty((H, nb, k_sel), **i32)
    prot = torch.empty((n_prot,), **i32)
    tail_lse = torch.empty((H, nb), **f32)
    tail_v = torch.empty((H, nb, D), **f32)
    ws_dense = ws(api.dense_tara_workspace_bytes(n, H, D, 1))
    ws_via = ws(api.via_workspace_bytes(seg, t, H, D, 1))
    ws_router = ws(api.router_tail_workspace_bytes(n, H, D))
    ws_sparse = ws(api.lib().attn_block_sparse_workspace(n, H, D, 1))
    ws_q8 = ws(api.int8qk_workspace_bytes(n, H, D))

    def step():
        api.attn_dense_tara(qd, kd, vd, seg_d, t_d, seg_d, t_d, *wl.tara, scale=wl.scale,
                            o=o_dense, lse=l_dense, ws=ws_dense)
        api.attn_dense_tara_via(qd, kd, vd, seg_d, t_d, seg, t, *wl.tara, scale=wl.scale,
                                o=o_via, lse=l_via, ws=ws_via)
        api.attn_block_router_tail(qd, kd, vd, seg_d, wl.protected_prefix_len, k_sel, n_prot,
                                   scale=wl.scale, tiles=tiles, prot=prot, tail_lse=tail_lse,
                                   tail_v=tail_v, ws=ws_router)
        api.attn_block_sparse_tail(qd, kd, vd, seg_d, t_d, tiles, prot, tail_lse, tail_v,
                                   *wl.tara, scale=wl.scale, o=o_sp, lse=l_sp, ws=ws_sparse)
        api.attn_block_sparse_int8qk(qd, kd, vd, seg_d, t_d, tiles, prot, tail_lse=tail_lse,
                                     tail_v=tail_v, strength=wl.tara[0], window=wl.tara[1],
                                     falloff=wl.tara[2], cap=wl.tara[3], scale=wl.scale,
                                     o=o_q8, lse=l_q8, ws=ws_q8)

    outs = [o_dense, l_dense, o_via, l_via, tiles, prot, tail_lse, tail_v, o_sp, l_sp, o_q8,
            l_q8]
    names = ["o_dense", "l_dense", "o_via", "l_via", "tiles", "prot", "tail_lse", "tail_v",
             "o_sparse", "l_sparse", "o_int8", "l_int8"]
    step()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]

    # warm up on a side stream, then capture the whole step into one graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
        print(f"replay {rep}: all {len(outs)} outputs equal the eager results", flush=True)
