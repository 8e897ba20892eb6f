"""Concurrent calls on separate HIP streams.

The library keeps no global state and each call works only in the buffers it is given,
so calls with separate outputs and workspaces may run at the same time on different
streams. Here dense TARA, the partition path and router + block-sparse attention run
concurrently on three side streams; every result must equal the sequential result on
the default stream bit for bit (the kernels are deterministic)."""
import pytest
import torch

from block_sparse_attention_02_amd import api, workloads as W
from gpu_common import layout_device, to_device

pytestmark = pytest.mark.gpu


def test_concurrent_streams_match_sequential():
    wl = W.custom("streams", [W.Span(W.SEG_TEXT, 70), W.Span(W.SEG_GUIDE, 8 * 120, 8),
                              W.Span(W.SEG_AUDIO, 33), W.Span(W.SEG_OUTPUT, 8 * 130, 8)],
                  heads=4, head_dim=128, dtype="bf16", seed_index=73, frame_weight=0.7,
                  protected_prefix_len=70)
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    n, H, D = qd.shape
    plan = api.router_plan(seg, 70, 0.7)
    print(f"case {wl.name} n={n} H={H} plan={plan}", flush=True)

    f32 = dict(dtype=torch.float32, device="cuda")

    def buffers():
        # every output and workspace exists before any launch and stays alive until the
        # final synchronisation (the caching allocator must not hand memory still in use
        # on a side stream to a later allocation)
        u8 = dict(dtype=torch.uint8, device="cuda")
        return dict(
            o1=torch.empty_like(qd), l1=torch.empty((n, H), **f32),
            o2=torch.empty_like(qd), l2=torch.empty((n, H), **f32),
            o3=torch.empty_like(qd), l3=torch.empty((n, H), **f32),
            tiles=torch.empty((H, plan["nb"], plan["k_sel"]), dtype=torch.int32, device="cuda"),
            prot=torch.empty((plan["n_prot"],), dtype=torch.int32, device="cuda"),
            ws_d=torch.empty(api.dense_tara_workspace_bytes(n, H, D, 1), **u8),
            ws_v=torch.empty(api.via_workspace_bytes(seg, t, H, D, 1), **u8),
            ws_r=torch.empty(api.router_workspace_bytes(n, H, D), **u8),
            ws_s=torch.empty(api.dense_tara_workspace_bytes(n, H, D, 1), **u8))

    def run(b, stream):
        api.attn_dense_tara(qd, kd, vd, seg_d, t_d, seg_d, t_d, *wl.tara, scale=wl.scale,
                            o=b["o1"], lse=b["l1"], ws=b["ws_d"], stream=stream[0])
        api.attn_dense_tara_via(qd, kd, vd, seg_d, t_d, seg, t, *wl.tara, scale=wl.scale,
                                o=b["o2"], lse=b["l2"], ws=b["ws_v"], stream=stream[1])
        api.attn_block_router(qd, kd, seg_d, 70, plan["k_sel"], plan["n_prot"],
                              tiles=b["tiles"], prot=b["prot"], ws=b["ws_r"], stream=stream[2])
        api.attn_block_sparse(qd, kd, vd, seg_d, t_d, b["tiles"], b["prot"], *wl.tara,
                              scale=wl.scale, o=b["o3"], lse=b["l3"], ws=b["ws_s"],
                              stream=stream[2])
        return [b[x] for x in ("o1", "l1", "o2", "l2", "tiles", "prot", "o3", "l3")]

    ref_bufs, got_bufs = buffers(), buffers()
    torch.cuda.synchronize()
    ref = run(ref_bufs, [None, None, None])
    torch.cuda.synchronize()
    side = [torch.cuda.Stream() for _ in range(3)]
    got = run(got_bufs, side)
    torch.cuda.synchronize()
    names = ["o_dense", "l_dense", "o_via", "l_via", "tiles", "prot", "o_sparse", "l_sparse"]
    for name, a, b in zip(names, got, ref):
        assert torch.equal(a, b), f"{name} differs between concurrent and sequential runs"
