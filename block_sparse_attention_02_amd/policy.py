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
- The other inputs of the table that choose a path map onto library calls:
  ``enabled`` (off = dense for a like-for-like baseline), ``dense_last_steps`` and
  ``dense_steps`` (sampling steps forced dense; the caller passes the step index),
  ``reference_protection`` (Off / Light / Heavy: the quota router), ``tail_correction``
  (the pooled tail key), ``use_int8_qk`` (the int8 QK product) and, from "H3 sparse-
  attention breakpoints", query blocks of sink segments that attend every key.

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
_REF_MODES = {"off": api.H3_REF_OFF, "light": api.H3_REF_LIGHT, "heavy": api.H3_REF_HEAVY}


def parse_steps(spec) -> frozenset:
    """Step indices from "0,1", "0-2", "0-2,5" or "" (none); a set of ints passes through."""
    if not isinstance(spec, str):
        return frozenset(int(s) for s in spec)
    out = set()
    for part in spec.replace(" ", "").split(","):
        if not part:
            continue
        if "-" in part:
            lo, hi = part.split("-", 1)
            lo, hi = int(lo), int(hi)
            if lo < 0 or hi < lo:
                raise ValueError(f"dense_steps: bad range {part!r}")
            out.update(range(lo, hi + 1))
        else:
            if int(part) < 0:
                raise ValueError(f"dense_steps: bad step {part!r}")
            out.add(int(part))
    return frozenset(out)


@dataclass(frozen=True)
class SparsePolicy:
    """Knobs of the block-sparse path ("H3 SLA Attention", inputs table).

    Combinations the library has no kernel for are rejected here: the tail term with a
    reference quota (the quota router writes no tail terms) and the int8 QK product at
    block size 32.
    """
    sparsity_ratio: float = 0.90
    block_size: int = 64
    protected_prefix_len: int = 0
    min_seq_len: int = MIN_SEQ_LEN_DEFAULT
    enabled: bool = True
    reference_protection: str = "off"
    tail_correction: bool = False
    use_int8_qk: bool = False
    sink_segments: tuple = ()
    dense_last_steps: int = 0
    dense_steps: object = ""

    def __post_init__(self):
        mode = str(self.reference_protection).lower().split()[0] if self.reference_protection \
            else "off"
        if mode not in _REF_MODES:
            raise ValueError(f"reference_protection must be Off, Light or Heavy, not "
                             f"{self.reference_protection!r}")
        object.__setattr__(self, "reference_protection", mode)
        object.__setattr__(self, "dense_steps", parse_steps(self.dense_steps))
        object.__setattr__(self, "sink_segments", tuple(int(s) for s in self.sink_segments))
        if self.block_size not in (32, 64, 128):
            raise ValueError(f"block_size must be 32, 64 or 128, not {self.block_size}")
        if not 0.0 <= self.sparsity_ratio < 1.0:
            raise ValueError(f"sparsity_ratio must lie in [0, 1), not {self.sparsity_ratio}")
        if self.dense_last_steps < 0:
            raise ValueError("dense_last_steps must be >= 0")
        if self.tail_correction and mode != "off":
            raise ValueError("tail_correction cannot be combined with reference_protection")
        if self.use_int8_qk and self.block_size == 32:
            raise ValueError("use_int8_qk needs block_size 64 or 128")
        if any(not 0 <= s < 8 for s in self.sink_segments):
            raise ValueError("sink_segments are segment ids 0..7")


def _dense_reason(policy, n, step, total_steps):
    if not policy.enabled:
        return "disabled"
    if policy.sparsity_ratio == 0.0:
        return "sparsity_ratio 0"
    if n < policy.min_seq_len:
        return f"{n} rows < min_seq_len {policy.min_seq_len}"
    if step is not None:
        if step in policy.dense_steps:
            return f"step {step} in dense_steps"
        if (policy.dense_last_steps and total_steps is not None
                and step >= total_steps - policy.dense_last_steps):
            return f"step {step} among the last {policy.dense_last_steps} of {total_steps}"
    return None


def attention(q, k, v, seg, t, seg_host, policy=SparsePolicy(), strength=2.0, window=0.20,
              falloff=0.25, cap=6.0, scale=None, o=None, lse=None, step=None,
              total_steps=None, ops=api):
    """TARA self-attention of one packed sequence through the path the policy picks.

    q, k, v [n, heads, head_dim], seg [n] and t [n] on the GPU; seg_host [n] is a host
    copy of seg (plans the routed tile counts without a device round trip). ``step`` and
    ``total_steps`` (optional) place the call in a sampling run for ``dense_steps`` and
    ``dense_last_steps``. Returns (o, lse, path). ``ops`` is the binding (api); tests may
    pass a stand-in.
    """
    n = int(q.shape[0])
    tara = (strength, window, falloff, cap)
    bs = policy.block_size
    reason = _dense_reason(policy, n, step, total_steps)
    path = "dense" if reason else None
    if path is None:
        try:
            tail_lse = tail_v = None
            if policy.reference_protection != "off":
                mode = _REF_MODES[policy.reference_protection]
                plan = ops.router_plan_ref(seg_host, policy.protected_prefix_len,
                                           policy.sparsity_ratio, mode, block_size=bs)
                tiles, prot = ops.attn_block_router_ref(q, k, seg, seg_host,
                                                        policy.protected_prefix_len,
                                                        policy.sparsity_ratio, mode,
                                                        block_size=bs)
            else:
                plan = ops.router_plan(seg_host, policy.protected_prefix_len,
                                       policy.sparsity_ratio, block_size=bs)
                if policy.tail_correction:
                    tiles, prot, tail_lse, tail_v = ops.attn_block_router_tail(
                        q, k, v, seg, policy.protected_prefix_len, plan["k_sel"],
                        plan["n_prot"], scale=scale, block_size=bs)
                else:
                    tiles, prot = ops.attn_block_router(q, k, seg, policy.protected_prefix_len,
                                                        plan["k_sel"], plan["n_prot"],
                                                        block_size=bs)
            tiles = tiles if plan["k_sel"] else None
            prot = prot if plan["n_prot"] else None
            sinks = sum(1 << s for s in policy.sink_segments)
            if policy.use_int8_qk:
                o, lse = ops.attn_block_sparse_int8qk(q, k, v, seg, t, tiles, prot, tail_lse,
                                                      tail_v, sinks, *tara, scale=scale,
                                                      block_size=bs, o=o, lse=lse)
            elif sinks or tail_lse is not None:
                o, lse = ops.attn_block_sparse_sinks(q, k, v, seg, t, tiles, prot, sinks,
                                                     tail_lse, tail_v, *tara, scale=scale,
                                                     block_size=bs, o=o, lse=lse)
            else:
                o, lse = ops.attn_block_sparse(q, k, v, seg, t, tiles, prot, *tara,
                                               scale=scale, block_size=bs, o=o, lse=lse)
            path = "block_sparse"
            extras = [x for x, on in (("reference " + policy.reference_protection,
                                       policy.reference_protection != "off"),
                                      ("tail", policy.tail_correction),
                                      ("int8 QK", policy.use_int8_qk),
                                      (f"sinks {list(policy.sink_segments)}", sinks)) if on]
            reason = (f"sparsity {policy.sparsity_ratio:.2f}, block {bs}, "
                      f"{plan['n_prot']} protected + {plan['k_sel']} routed of {plan['nb']} "
                      "tiles" + "".join(", " + x for x in extras))
        except ops.H3Error as e:
            log.warning("h3attn: %s returned status %d (%s); falling back to dense TARA",
                        e.func, e.status, ops.status_string(e.status))
            path, reason = "dense_fallback", f"{e.func} status {e.status}"
    if path != "block_sparse":
        o, lse = ops.attn_dense_tara(q, k, v, seg, t, seg, t, *tara, scale=scale, o=o, lse=lse)
    log.info("h3attn: path=%s rows=%d heads=%d (%s)", path, n, int(q.shape[1]), reason)
    return o, lse, path
