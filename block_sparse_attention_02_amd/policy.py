"""Caller policy around the library: which path runs, and the dense fallback.

A dispatcher with no arithmetic of its own; every computation is a library call.
From "H3 SLA Attention":
- "The inputs that matter" and the inputs table (min_seq_len): sequences shorter than
  ``min_seq_len`` stay dense (they guard short attention calls where block selection
  costs more than it saves); sparsity 0 disables sparsity.
- "Install": when the sparse kernel fails, the call degrades to plain dense attention
  instead of failing the run, and the console says so.
- The inputs table's default for ``min_seq_len`` is 12228 (the prose of the same page
  says 8192; the table's value is taken, and both workloads here are far longer).

Every call logs one line on the ``h3attn`` logger naming the path that ran
(``dense``, ``block_sparse`` or ``dense_fallback``), and a warning with the failing
entry point and status before a fallback. The library's failure-injection hook
(environment variable ``H3ATTN_FORCE_FAIL=router|sparse|dense``) exercises the
fallback.
"""
from __future__ import annotations

import logging
from dataclasses import dataclass

from . import api

log = logging.getLogger("h3attn")

MIN_SEQ_LEN_DEFAULT = 12228


@dataclass(frozen=True)
class SparsePolicy:
    """Knobs of the block-sparse path ("H3 SLA Attention", inputs table)."""
    sparsity_ratio: float = 0.90
    block_size: int = 64
    protected_prefix_len: int = 0
    min_seq_len: int = MIN_SEQ_LEN_DEFAULT


def attention(q, k, v, seg, t, seg_host, policy=SparsePolicy(), strength=2.0, window=0.20,
              falloff=0.25, cap=6.0, scale=None, o=None, lse=None, ops=api):
    """TARA self-attention of one packed sequence through the path the policy picks.

    q, k, v [n, heads, head_dim], seg [n] and t [n] on the GPU; seg_host [n] is a host
    copy of seg (plans the routed tile counts without a device round trip). Returns
    (o, lse, path). ``ops`` is the binding (api); tests may pass a stand-in.
    """
    n = int(q.shape[0])
    tara = (strength, window, falloff, cap)
    path, reason = None, ""
    if policy.sparsity_ratio == 0.0:
        path, reason = "dense", "sparsity_ratio 0"
    elif n < policy.min_seq_len:
        path, reason = "dense", f"{n} rows < min_seq_len {policy.min_seq_len}"
    if path is None:
        try:
            plan = ops.router_plan(seg_host, policy.protected_prefix_len, policy.sparsity_ratio,
                                   block_size=policy.block_size)
            tiles, prot = ops.attn_block_router(q, k, seg, policy.protected_prefix_len,
                                                plan["k_sel"], plan["n_prot"],
                                                block_size=policy.block_size)
            o, lse = ops.attn_block_sparse(q, k, v, seg, t, tiles if plan["k_sel"] else None,
                                           prot if plan["n_prot"] else None, *tara,
                                           scale=scale, block_size=policy.block_size, o=o,
                                           lse=lse)
            path = "block_sparse"
            reason = (f"sparsity {policy.sparsity_ratio:.2f}, block {policy.block_size}, "
                      f"{plan['n_prot']} protected + {plan['k_sel']} routed of {plan['nb']} "
                      "tiles")
        except ops.H3Error as e:
            log.warning("h3attn: %s returned status %d (%s); falling back to dense TARA",
                        e.func, e.status, ops.status_string(e.status))
            path, reason = "dense_fallback", f"{e.func} status {e.status}"
    if path != "block_sparse":
        o, lse = ops.attn_dense_tara(q, k, v, seg, t, seg, t, *tara, scale=scale, o=o, lse=lse)
    log.info("h3attn: path=%s rows=%d heads=%d (%s)", path, n, int(q.shape[1]), reason)
    return o, lse, path
