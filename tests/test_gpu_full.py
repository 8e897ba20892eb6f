"""GPU parity at the full 116,883-row x 56-head size, in the same launch
configuration the benchmark times.
- Router: every tile list of all 56 heads bit-exact against the oracle, at each
  sparsity of the sweep (block 64) and at blocks of 32 and 128 (s = 0.90).
- Outputs: sampled rows the oracle computes one by one, 3 heads x 8 fixed query
  blocks (segment boundaries and the 19-row tail) plus 16 seeded random blocks.
  The oracle attends with its own tile lists, after the GPU lists were checked
  equal to them."""
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_02_amd import api, workloads as W
from gpu_common import checked_routes, checked_routes_ref, compare, f64, to_device

pytestmark = pytest.mark.gpu

HEADS = [0, 27, 55]
FIXED_BLOCKS = [0, 113, 500, 962, 970, 977, 1400, 1826]
ORACLE_THREADS = 16


def _blocks():
    rng = np.random.default_rng(2024)
    extra = [b for b in rng.permutation(1827).tolist() if b not in FIXED_BLOCKS][:16]
    return sorted(FIXED_BLOCKS + extra)


def _oracle_lists(q32, k32, seg, prefix, bs, ks):
    """The oracle's routing of one head for several routed counts: route_head's steps
    (block means, pooled scores over the video tiles, top-k), with the pooled scores
    formed once for all counts in ``ks``. Returns {k: [nb, k] tile lists}."""
    _, _, video, _ = oracle.router_plan(seg, prefix, bs, 0.0)
    qbar = oracle.block_means_fp32(q32, bs)
    kbar = oracle.block_means_fp32(k32, bs)
    scores = oracle.pooled_scores_fp32(qbar, kbar[video])
    return {kk: oracle.select_topk(scores, video, kk) for kk in ks}


def _all_heads_mismatches(q, k, seg, prefix, bs, got):
    """Mismatching (head, query block) tile lists of every head: ``got`` maps each routed
    count k to the GPU lists [H, nb, k]. Heads run in a thread pool (numpy releases the
    GIL inside its array operations)."""
    H = q.shape[1]

    def one(h):
        ref = _oracle_lists(W.to_float32(q[:, h], "bf16"), W.to_float32(k[:, h], "bf16"), seg,
                            prefix, bs, list(got))
        return {kk: int(np.sum(np.any(got[kk][h] != ref[kk], axis=1))) for kk in got}

    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        per_head = list(ex.map(one, range(H)))
    return {kk: sum(m[kk] for m in per_head) for kk in got}


@pytest.fixture(scope="module")
def full():
    wl = W.FULL_SPARSE
    t0 = time.time()
    q, k, v = W.make_qkv(wl)
    print(f"inputs generated in {time.time() - t0:.1f}s", flush=True)
    seg, t = W.layout(wl)
    dev = dict(q=to_device(q, "bf16"), k=to_device(k, "bf16"), v=to_device(v, "bf16"),
               seg=torch.from_numpy(seg).cuda(), t=torch.from_numpy(t).cuda())
    host = {n: f64(x[:, HEADS], "bf16") for n, x in (("q", q), ("k", k), ("v", v))}
    host32 = {n: W.to_float32(x[:, HEADS], "bf16") for n, x in (("q", q), ("k", k))}
    return wl, seg, t, dev, host, host32, (q, k, v)


def _sample_rows(blocks, n):
    return np.concatenate([np.arange(b * 64, min(n, b * 64 + 64)) for b in blocks])


def _dense_ref(wl, seg, t, host, rows):
    o, l = oracle.dense_tara(host["q"][rows], host["k"], host["v"], seg[rows], t[rows], seg, t,
                             wl.tara, wl.scale)
    return o, l


def test_full_dense_direct_sampled(full):
    wl, seg, t, dev, host, _, _ = full
    print("dense direct 116883 x 56", flush=True)
    o, lse = api.attn_dense_tara(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"], dev["seg"],
                                 dev["t"], *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(_blocks(), wl.n)
    o_ref, l_ref = _dense_ref(wl, seg, t, host, rows)
    ri = torch.from_numpy(rows).cuda()
    compare(o[ri][:, HEADS], lse[ri][:, HEADS], o_ref, l_ref, "bf16", "full dense direct")


def test_full_dense_via_sampled(full):
    wl, seg, t, dev, host, _, _ = full
    print("dense via partitions 116883 x 56", flush=True)
    o, lse = api.attn_dense_tara_via(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"], seg, t,
                                     *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(_blocks(), wl.n)
    o_ref, l_ref = _dense_ref(wl, seg, t, host, rows)
    ri = torch.from_numpy(rows).cuda()
    compare(o[ri][:, HEADS], lse[ri][:, HEADS], o_ref, l_ref, "bf16", "full dense via")


@pytest.mark.parametrize("sparsity", [0.90, 0.50, 0.70, 0.85, 0.95])
def test_full_router_and_sparse_sampled(full, sparsity):
    wl, seg, t, dev, host, host32, raw = full
    plan = api.router_plan(seg, wl.protected_prefix_len, sparsity)
    assert plan["n_prot"] == 130 and plan["n_video"] == 1697
    print(f"router + sparse s={sparsity} k={plan['k_sel']}", flush=True)
    tiles, prot = api.attn_block_router(dev["q"], dev["k"], dev["seg"], wl.protected_prefix_len,
                                        plan["k_sel"], plan["n_prot"])
    o, lse = api.attn_block_sparse(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"], tiles,
                                   prot, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    tl, pr = checked_routes(tiles, prot, wl, raw[0], raw[1], seg, plan["k_sel"], HEADS,
                            tag=f"full s={sparsity}")
    blocks = _blocks()
    ref = oracle.block_sparse(host["q"], host["k"], host["v"], seg, t, wl.tara, wl.scale, 64, pr,
                              tl, heads=range(len(HEADS)), qblocks=blocks)
    og, lg, orf, lrf = [], [], [], []
    for (j, qb), (ob, lb) in ref.items():
        lo, hi = qb * 64, min(wl.n, qb * 64 + 64)
        og.append(o[lo:hi, HEADS[j]])
        lg.append(lse[lo:hi, HEADS[j]])
        orf.append(ob)
        lrf.append(lb)
    compare(torch.cat(og), torch.cat(lg), np.concatenate(orf), np.concatenate(lrf), "bf16",
            f"full sparse s={sparsity}")


def test_full_router_all_heads_bit_exact(full):
    """Every tile list of all 56 heads x 1,827 query blocks against the oracle at each
    sparsity of the sweep (block 64), and the protected list."""
    wl, seg, t, dev, host, host32, raw = full
    got = {}
    for sparsity in wl.sparsities:
        plan = api.router_plan(seg, wl.protected_prefix_len, sparsity)
        tiles, prot = api.attn_block_router(dev["q"], dev["k"], dev["seg"],
                                            wl.protected_prefix_len, plan["k_sel"],
                                            plan["n_prot"])
        torch.cuda.synchronize()
        _, prot_ref, _, _ = oracle.router_plan(seg, wl.protected_prefix_len, 64, sparsity)
        assert np.array_equal(prot.cpu().numpy(), prot_ref)
        got[plan["k_sel"]] = tiles.cpu().numpy()
    print(f"router all heads, k = {sorted(got)}", flush=True)
    # the shared-scores helper is route_head's composition: check it on one head and count
    q32, k32 = W.to_float32(raw[0][:, 55], "bf16"), W.to_float32(raw[1][:, 55], "bf16")
    assert np.array_equal(_oracle_lists(q32, k32, seg, wl.protected_prefix_len, 64, [170])[170],
                          oracle.route_head(q32, k32, seg, wl.protected_prefix_len, 64, 170))
    t0 = time.time()
    mism = _all_heads_mismatches(raw[0], raw[1], seg, wl.protected_prefix_len, 64, got)
    print(f"oracle lists of 56 heads in {time.time() - t0:.1f}s; mismatching lists per k: "
          f"{mism}", flush=True)
    assert all(m == 0 for m in mism.values())


@pytest.mark.parametrize("bs", [32, 128])
def test_full_router_all_heads_block_sizes(full, bs):
    """Every tile list of all 56 heads at blocks of 32 and 128 rows, s = 0.90."""
    wl, seg, t, dev, host, host32, raw = full
    plan = api.router_plan(seg, wl.protected_prefix_len, 0.90, block_size=bs)
    tiles, prot = api.attn_block_router(dev["q"], dev["k"], dev["seg"], wl.protected_prefix_len,
                                        plan["k_sel"], plan["n_prot"], block_size=bs)
    torch.cuda.synchronize()
    _, prot_ref, _, _ = oracle.router_plan(seg, wl.protected_prefix_len, bs, 0.90)
    assert np.array_equal(prot.cpu().numpy(), prot_ref)
    print(f"router all heads bs={bs} k={plan['k_sel']}", flush=True)
    t0 = time.time()
    mism = _all_heads_mismatches(raw[0], raw[1], seg, wl.protected_prefix_len, bs,
                                 {plan["k_sel"]: tiles.cpu().numpy()})
    print(f"oracle lists of 56 heads (bs={bs}) in {time.time() - t0:.1f}s; mismatching "
          f"lists: {mism}", flush=True)
    assert all(m == 0 for m in mism.values())


@pytest.mark.parametrize("mode", [1, 2])
def test_full_reference_protection(full, mode):
    """Full scale, s = 0.90, Light (the guide range keeps its best 128 of 848 tiles on top of
    the ordinary 170) or Heavy (all 848 guide tiles protected, 85 of the 849 output tiles
    routed): every list of all 56 heads bit-exact, sampled outputs against the oracle over
    its own lists."""
    wl, seg, t, dev, host, host32, raw = full
    plan = api.router_plan_ref(seg, wl.protected_prefix_len, 0.90, mode)
    print(f"router ref mode={mode} 116883 x 56, plan={plan}", flush=True)
    tiles, prot = api.attn_block_router_ref(dev["q"], dev["k"], dev["seg"], seg,
                                            wl.protected_prefix_len, 0.90, mode)
    o, lse = api.attn_block_sparse(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"], tiles,
                                   prot, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    got = tiles.cpu().numpy()
    t0 = time.time()

    def one(h):
        ref = oracle.route_head_ref(W.to_float32(raw[0][:, h], "bf16"),
                                    W.to_float32(raw[1][:, h], "bf16"), seg,
                                    wl.protected_prefix_len, 64, 0.90, mode)
        return int(np.sum(np.any(got[h] != ref, axis=1)))

    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        mism = sum(ex.map(one, range(wl.heads)))
    print(f"oracle lists of 56 heads in {time.time() - t0:.1f}s; mismatching: {mism}",
          flush=True)
    assert mism == 0
    tl, pr = checked_routes_ref(tiles, prot, wl, raw[0], raw[1], seg, 0.90, mode, HEADS,
                                tag=f"full ref mode={mode}")
    blocks = _blocks()
    ref = oracle.block_sparse(host["q"], host["k"], host["v"], seg, t, wl.tara, wl.scale, 64, pr,
                              tl, heads=range(len(HEADS)), qblocks=blocks)
    og, lg, orf, lrf = [], [], [], []
    for (j, qb), (ob, lb) in ref.items():
        lo, hi = qb * 64, min(wl.n, qb * 64 + 64)
        og.append(o[lo:hi, HEADS[j]])
        lg.append(lse[lo:hi, HEADS[j]])
        orf.append(ob)
        lrf.append(lb)
    compare(torch.cat(og), torch.cat(lg), np.concatenate(orf), np.concatenate(lrf), "bf16",
            f"full sparse ref mode={mode}")


# ------------------------------------------------------------------ isolated shape
# The isolated attention shape of the Flash Partitions page (107,126 rows x 8 heads),
# direct and through the partition path, in the launch configuration the benchmark
# times; sampled rows against the oracle.
P1_HEADS = [0, 7]
P1_BLOCKS = [0, 80, 400, 867, 880, 886, 1300, 1673]  # text/guide, guide/audio, audio/output, tail


@pytest.fixture(scope="module")
def micro():
    wl = W.P1_MICRO
    q, k, v = W.make_qkv(wl)
    seg, t = W.layout(wl)
    dev = dict(q=to_device(q, "bf16"), k=to_device(k, "bf16"), v=to_device(v, "bf16"),
               seg=torch.from_numpy(seg).cuda(), t=torch.from_numpy(t).cuda())
    host = {n: f64(x[:, P1_HEADS], "bf16") for n, x in (("q", q), ("k", k), ("v", v))}
    return wl, seg, t, dev, host


@pytest.mark.parametrize("path", ["direct", "via"])
def test_p1_shape_dense_tara_sampled(micro, path):
    wl, seg, t, dev, host = micro
    print(f"case {wl.name} path={path}", flush=True)
    if path == "direct":
        o, lse = api.attn_dense_tara(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"],
                                     dev["seg"], dev["t"], *wl.tara, scale=wl.scale)
    else:
        o, lse = api.attn_dense_tara_via(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"], seg, t,
                                         *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(P1_BLOCKS, wl.n)
    o_ref, l_ref = _dense_ref(wl, seg, t, host, rows)
    ri = torch.from_numpy(rows).cuda()
    compare(o[ri][:, P1_HEADS], lse[ri][:, P1_HEADS], o_ref, l_ref, "bf16", f"p1 shape {path}")


@pytest.mark.parametrize("sparsity", [0.90, 0.95])
def test_full_sparse_with_tail_sampled(full, sparsity):
    """Full scale, TARA on routed guide tiles plus the pooled tail key (at s = 0.95 the
    tail key carries the largest share of a row's weight): tail terms of the sampled heads
    against the oracle, outputs on sampled rows."""
    wl, seg, t, dev, host, host32, raw = full
    plan = api.router_plan(seg, wl.protected_prefix_len, sparsity)
    print(f"router + tail 116883 x 56, s={sparsity}", flush=True)
    tiles, prot, tl, tv = api.attn_block_router_tail(dev["q"], dev["k"], dev["v"], dev["seg"],
                                                     wl.protected_prefix_len, plan["k_sel"],
                                                     plan["n_prot"], scale=wl.scale)
    o, lse = api.attn_block_sparse_tail(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"], tiles,
                                        prot, tl, tv, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    tl_ref, pr = checked_routes(tiles, prot, wl, raw[0], raw[1], seg, plan["k_sel"], HEADS,
                                tag=f"full tail s={sparsity}")
    tails = {}
    for j, h in enumerate(HEADS):
        tails[j] = oracle.tail_terms(host32["q"][:, j], host32["k"][:, j], host["v"][:, j], seg,
                                     wl.protected_prefix_len, 64, tl_ref[j], wl.scale)
        fin = np.isfinite(tails[j][0])
        el = float(np.max(np.abs(tl[h].cpu().numpy()[fin] - tails[j][0][fin])))
        ev = float(np.max(np.abs(tv[h].cpu().numpy() - tails[j][1])))
        print(f"[full tail terms head {h}] lse err {el:.2e} v err {ev:.2e}", flush=True)
        assert el < 1e-3 and ev < 1e-3
    blocks = _blocks()
    ref = oracle.block_sparse(host["q"], host["k"], host["v"], seg, t, wl.tara, wl.scale, 64,
                              pr, tl_ref, heads=range(3), qblocks=blocks, tails=tails)
    og, lg, orf, lrf = [], [], [], []
    for (j, qb), (ob, lb) in ref.items():
        lo, hi = qb * 64, min(wl.n, qb * 64 + 64)
        og.append(o[lo:hi, HEADS[j]])
        lg.append(lse[lo:hi, HEADS[j]])
        orf.append(ob)
        lrf.append(lb)
    compare(torch.cat(og), torch.cat(lg), np.concatenate(orf), np.concatenate(lrf), "bf16",
            f"full sparse tail s={sparsity}")


@pytest.mark.parametrize("bs", [32, 128])
def test_full_block_sizes_with_audio_sinks_sampled(full, bs):
    """Full scale, s = 0.90, blocks of 32 or 128 rows, TARA on routed guide tiles, audio
    sink query blocks dense: router lists of the sampled heads bit-exact, outputs of
    sampled blocks (segment boundaries, the audio span, the ragged tail) against the
    oracle."""
    wl, seg, t, dev, host, host32, raw = full
    plan = api.router_plan(seg, wl.protected_prefix_len, 0.90, block_size=bs)
    print(f"router + sparse + audio sinks bs={bs} k={plan['k_sel']}", flush=True)
    tiles, prot = api.attn_block_router(dev["q"], dev["k"], dev["seg"], wl.protected_prefix_len,
                                        plan["k_sel"], plan["n_prot"], block_size=bs)
    o, lse = api.attn_block_sparse_sinks(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"],
                                         tiles, prot, 1 << W.SEG_AUDIO, None, None, *wl.tara,
                                         scale=wl.scale, block_size=bs)
    torch.cuda.synchronize()
    tl, pr = checked_routes(tiles, prot, wl, raw[0], raw[1], seg, plan["k_sel"], HEADS, bs=bs,
                            tag=f"full bs={bs}")
    nb = plan["nb"]
    # blocks holding rows 0, 7258/7259 (text/guide), 61570/61571 (guide/audio), 62000
    # (audio), 62570/62571 (audio/output), 90000 and the last row
    blocks = sorted({r // bs for r in (0, 7258, 7259, 61570, 61571, 62000, 62570, 62571,
                                       90000, wl.n - 1)})
    ref = oracle.block_sparse(host["q"], host["k"], host["v"], seg, t, wl.tara, wl.scale, bs, pr,
                              tl, heads=range(len(HEADS)), qblocks=blocks,
                              sink_segments=(W.SEG_AUDIO,))
    og, lg, orf, lrf = [], [], [], []
    for (j, qb), (ob, lb) in ref.items():
        lo, hi = qb * bs, min(wl.n, qb * bs + bs)
        og.append(o[lo:hi, HEADS[j]])
        lg.append(lse[lo:hi, HEADS[j]])
        orf.append(ob)
        lrf.append(lb)
    assert blocks[-1] == nb - 1
    compare(torch.cat(og), torch.cat(lg), np.concatenate(orf), np.concatenate(lrf), "bf16",
            f"full sparse bs={bs} audio sinks")


def test_full_sparse_int8qk_sampled(full):
    """Full scale, s = 0.90, block 64, TARA on routed guide tiles, int8 QK product:
    sampled rows against the oracle's attention on the dequantized q and k."""
    wl, seg, t, dev, host, host32, raw = full
    plan = api.router_plan(seg, wl.protected_prefix_len, 0.90)
    print("router + int8 QK sparse 116883 x 56, s=0.90", flush=True)
    tiles, prot = api.attn_block_router(dev["q"], dev["k"], dev["seg"], wl.protected_prefix_len,
                                        plan["k_sel"], plan["n_prot"])
    o, lse = api.attn_block_sparse_int8qk(dev["q"], dev["k"], dev["v"], dev["seg"], dev["t"],
                                          tiles, prot, None, None, 0, *wl.tara, scale=wl.scale)
    torch.cuda.synchronize()
    tl, pr = checked_routes(tiles, prot, wl, raw[0], raw[1], seg, plan["k_sel"], HEADS,
                            tag="full int8")
    blocks = _blocks()
    ref = oracle.block_sparse(host["q"], host["k"], host["v"], seg, t, wl.tara, wl.scale, 64,
                              pr, tl, heads=range(len(HEADS)), qblocks=blocks, int8_qk=True)
    og, lg, orf, lrf = [], [], [], []
    for (j, qb), (ob, lb) in ref.items():
        lo, hi = qb * 64, min(wl.n, qb * 64 + 64)
        og.append(o[lo:hi, HEADS[j]])
        lg.append(lse[lo:hi, HEADS[j]])
        orf.append(ob)
        lrf.append(lb)
    compare(torch.cat(og), torch.cat(lg), np.concatenate(orf), np.concatenate(lrf), "bf16",
            "full sparse int8 QK s=0.9")
