"""The allocation-free router entry point (attn_block_router_static): its scratch is the
library's static device array, so the call takes no workspace. Its tile and protected
lists must equal attn_block_router's bit for bit, on consecutive calls that share the
array, the second with a smaller input (stale contents of the first must not leak), and
a problem larger than the array is rejected before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

from block_sparse_attention_02_amd import api, workloads as W
from gpu_common import layout_device, to_device

pytestmark = pytest.mark.gpu


def _compare(wl, sparsity, bs):
    seg, t, seg_d, t_d = layout_device(wl)
    q, k, _ = W.make_qkv(wl)
    qd, kd = to_device(q, wl.dtype), to_device(k, wl.dtype)
    plan = api.router_plan(seg, wl.protected_prefix_len, sparsity, block_size=bs)
    print(f"case static router {wl.name} n={wl.n} H={wl.heads} d={wl.head_dim} {wl.dtype} "
          f"bs={bs} plan={plan}", flush=True)
    tw, pw = api.attn_block_router(qd, kd, seg_d, wl.protected_prefix_len, plan["k_sel"],
                                   plan["n_prot"], block_size=bs)
    ts, ps = api.attn_block_router_static(qd, kd, seg_d, wl.protected_prefix_len, plan["k_sel"],
                                          plan["n_prot"], block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(tw, ts) and torch.equal(pw, ps), wl.name
    return ts


def test_static_scratch_router_matches_workspace_router():
    small = W.custom("static_small", [W.Span(W.SEG_TEXT, 70), W.Span(W.SEG_GUIDE, 6 * 90, 6),
                                      W.Span(W.SEG_AUDIO, 25), W.Span(W.SEG_OUTPUT, 6 * 90 + 7, 6)],
                     heads=3, head_dim=64, dtype="f32", seed_index=160, frame_weight=0.7,
                     protected_prefix_len=70)
    _compare(W.MID_SPARSE, 0.85, 64)      # 31,552 rows x 24 heads
    _compare(small, 0.5, 32)              # then a smaller call on the same array
    _compare(small, 0.9, 128)


def test_static_scratch_holds_the_full_scale_router():
    need = api.router_workspace_bytes(116883, 56, 128, 64)
    assert need <= api.H3_STATIC_SCRATCH_BYTES, need


def test_static_scratch_rejects_a_larger_problem():
    """896,000 rows x 56 heads needs 0.8 GB of router scratch: H3_ESCRATCH, returned before
    any HIP call (the placeholder pointers are never read)."""
    P = ctypes.c_void_p(4096)
    assert api.router_workspace_bytes(896000, 56, 128, 64) > api.H3_STATIC_SCRATCH_BYTES
    st = api.lib().attn_block_router_static(P, P, 1, 896000, 56, 128, P, 0, 64, 10, P, P, 1, None)
    assert st == api.H3_ESCRATCH
    assert "static scratch" in api.status_string(st)
