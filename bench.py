"""Benchmark of the TARA dense / block-sparse attention hot path on one MI355X.

One step = one pass of the whole hot path over the full-scale packed sequence
(116,883 rows x 56 heads x d 128, bf16, inputs resident in HBM):
  1. dense TARA attention, one direct call (attn_dense_tara);
  2. block-sparse attention at sparsity 0.90: router (attn_block_router) +
     sparse attention (attn_block_sparse) with the TARA penalty on routed
     guide tiles;
  3. dense TARA through the positive-partition decomposition with LSE merges
     (attn_dense_tara_via).
``value`` is the dense TARA call's dense-equivalent throughput,
4*N^2*d*H = 391.71 TFLOP over its median ms/call (HIP events on the launch
stream); ``ms_per_step`` is the wall time of the whole step. The block-sparse
call is reported as router + sparse ms and its speed-up over the dense call
(its executed work is a fraction of the dense work, so it is not folded into a
dense-equivalent rate), the partition path as ms and dense-equivalent TFLOP/s.
Beside them: a sparsity sweep, the roofline of the dominant kernel (the dense
TARA attention kernel) and the float64 CPU oracle timed on a sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "ms/call + dense-equiv TFLOP/s (%MFMA peak), 116,883 rows x 56 heads, 1 GPU"
DENSE_KERNEL = "attn_bf16_kernel<128, false, true, false, false>"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_bf16_dense_tara_116883x56_pmc.json")


def code_hash(text):
    """Hash of the code lines of a HIP source: // comments and blank lines do not count, so
    a comment edit leaves the compiled kernel, and its counter summary, valid."""
    h = hashlib.sha256()
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def kernel_source_hash():
    with open(os.path.join(ROOT, "block_sparse_attention_02_amd", "csrc", "attn_bf16.hip")) as f:
        return code_hash(f.read())


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--sparsity", type=float, default=0.90)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["all", "dense", "sparse", "via"], default="all",
                    help="profiling aid: run one row of the step only (the JSON line then "
                         "covers that row)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="profiling aid: only run a plain 1 GiB device-to-device copy, whose "
                         "FETCH_SIZE/WRITE_SIZE readings scale the HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                       "COPY_WRITE_DIR"),
                    help="CPU only: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of "
                         "the dense kernel and of the calibration copy into the per-launch "
                         "HBM traffic summary under profiles/")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration():
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}))


def _counter_kib(path, counter, kernel_substr):
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for '{kernel_substr}' under {path}")
    return float(np.mean(vals)), len(vals)


DENSE_ONLY = "python3 bench.py --only dense --steps 1 --warmup 0 --no-cpu --no-sweep"


def pmc_summary(dirs):
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    kern = DENSE_KERNEL
    copy_kern = "copyBuffer"
    f_kib, nf = _counter_kib(fetch_dir, "FETCH_SIZE", kern)
    w_kib, nw = _counter_kib(write_dir, "WRITE_SIZE", kern)
    cf_kib, _ = _counter_kib(cfetch_dir, "FETCH_SIZE", copy_kern)
    cw_kib, _ = _counter_kib(cwrite_dir, "WRITE_SIZE", copy_kern)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    fetch = f_kib * 1024.0 * f_scale
    write = w_kib * 1024.0 * w_scale
    out = {"kernel": kern, "workload": "dense TARA 116,883 x 56 x 128 bf16",
           "source_hash": kernel_source_hash(),
           "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
           "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib, "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": fetch + write,
           "launches_averaged": [nf, nw],
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- {DENSE_ONLY}",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- {DENSE_ONLY}",
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cfetch_dir} -o run -- "
               "python3 bench.py --copy-calibration",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cwrite_dir} -o run -- "
               "python3 bench.py --copy-calibration",
               f"python3 bench.py --pmc-summary {fetch_dir} {write_dir} {cfetch_dir} {cwrite_dir}"]}
    with open(PMC_SUMMARY, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def cpu_baseline(wl, q, k, v, seg, t):
    """The float64 oracle on a bounded sample of the same workload."""
    import oracle
    from block_sparse_attention_02_amd import workloads as W
    threads = len(os.sched_getaffinity(0))
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            threads = min(threads, int(os.environ[var]))
            break
    # about 15 s of float64 work on 16 cores: 3 heads x ~135 query blocks spread over
    # the sequence, including every segment boundary and the ragged last block
    heads = [0, 27, 55]
    nb = (wl.n + 63) // 64
    blocks = sorted(set(range(0, nb, 14)) | {113, 962, 970, 977, nb - 1})
    rows = np.concatenate([np.arange(b * 64, min(wl.n, b * 64 + 64)) for b in blocks])
    q64 = W.to_float64(q[rows][:, heads], "bf16")
    k64 = W.to_float64(k[:, heads], "bf16")
    v64 = W.to_float64(v[:, heads], "bf16")
    t0 = time.perf_counter()
    oracle.dense_tara(q64, k64, v64, seg[rows], t[rows], seg, t, wl.tara, wl.scale)
    dt = time.perf_counter() - t0
    flops = 4.0 * len(rows) * wl.n * wl.head_dim * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 dense TARA oracle, {len(rows)} query rows x {wl.n} keys x "
                      f"{len(heads)} heads ({flops / 1e12:.3f} dense TFLOP) in {dt:.1f} s"}


def call_summaries(rows, dense_flop, sparsity, k_sel, n_prot, kept):
    """Per-call figures from the HIP-event times (ms) of the timed steps: medians, the
    dense-equivalent rate of the two full-attention calls, and the block-sparse call as
    router + sparse ms with its speed-up over the dense call."""
    def summary(name):
        xs = rows.get(name) or []
        if not xs:
            return None
        return {"ms": float(np.median(xs)), "ms_mean": float(np.mean(xs)), "n": len(xs)}

    calls = {}
    d = summary("dense")
    if d:
        tf = dense_flop / (d["ms"] * 1e-3) / 1e12
        calls["dense_tara"] = dict(d, dense_equiv_tflops=tf, frac_peak=tf / PEAK_BF16_TFLOPS)
    r, s = summary("router"), summary("sparse")
    if r and s:
        tot = r["ms"] + s["ms"]
        calls["block_sparse"] = {
            "sparsity": sparsity, "k_sel": k_sel, "n_prot": n_prot, "kept_frac": kept,
            "router_ms": r["ms"], "sparse_ms": s["ms"], "ms": tot,
            "executed_tflops": kept * dense_flop / (s["ms"] * 1e-3) / 1e12,
            "speedup_vs_dense": (d["ms"] / tot) if d else None,
            "target_speedup": 0.8 / kept,
        }
    vi = summary("via")
    if vi:
        tf = dense_flop / (vi["ms"] * 1e-3) / 1e12
        calls["dense_tara_via"] = dict(vi, dense_equiv_tflops=tf, frac_peak=tf / PEAK_BF16_TFLOPS)
    return calls


def headline_value(calls):
    """``value``: the dense TARA call's dense-equivalent TFLOP/s (None on a profiling run
    that leaves the dense call out)."""
    d = calls.get("dense_tara")
    return d["dense_equiv_tflops"] if d else None


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; the attention would "
                                   "shard by head across GPUs, which is not built here",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from block_sparse_attention_02_amd import api, workloads as W

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    wl = W.FULL_SPARSE
    N, H, D = wl.n, wl.heads, wl.head_dim
    dense_flop = 4.0 * N * N * D * H
    t0 = time.time()
    q, k, v = W.make_qkv(wl)
    seg, t = W.layout(wl)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()

    qd, kd, vd = dev(q), dev(k), dev(v)
    segd, td = torch.from_numpy(seg).cuda(), torch.from_numpy(t).cuda()
    scale = wl.scale
    tara = wl.tara
    plan = api.router_plan(seg, wl.protected_prefix_len, args.sparsity)
    k_sel, n_prot, nb = plan["k_sel"], plan["n_prot"], plan["nb"]
    kept = (n_prot + k_sel) / nb

    # every buffer allocated up front: the timed region only launches kernels
    o_dense = torch.empty_like(qd)
    l_dense = torch.empty((N, H), dtype=torch.float32, device="cuda")
    ws_dense = torch.empty(api.dense_tara_workspace_bytes(N, H, D, 1), dtype=torch.uint8,
                           device="cuda")
    tiles = torch.empty((H, nb, k_sel), dtype=torch.int32, device="cuda")
    prot = torch.empty((n_prot,), dtype=torch.int32, device="cuda")
    ws_router = torch.empty(api.router_workspace_bytes(N, H, D), dtype=torch.uint8, device="cuda")
    o_sparse = torch.empty_like(qd)
    l_sparse = torch.empty((N, H), dtype=torch.float32, device="cuda")
    o_via = torch.empty_like(qd)
    l_via = torch.empty((N, H), dtype=torch.float32, device="cuda")
    ws_via = torch.empty(api.via_workspace_bytes(seg, t, H, D, 1), dtype=torch.uint8,
                         device="cuda")

    stream = torch.cuda.current_stream()
    rows = {"dense": [], "router": [], "sparse": [], "via": []}

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(record):
        marks = []
        if args.only in ("all", "dense"):
            a = ev()
            api.attn_dense_tara(qd, kd, vd, segd, td, segd, td, *tara, scale=scale, o=o_dense,
                                lse=l_dense, ws=ws_dense)
            marks.append(("dense", a, ev()))
        if args.only in ("all", "sparse"):
            a = ev()
            api.attn_block_router(qd, kd, segd, wl.protected_prefix_len, k_sel, n_prot,
                                  tiles=tiles, prot=prot, ws=ws_router)
            b = ev()
            api.attn_block_sparse(qd, kd, vd, segd, td, tiles, prot, *tara, scale=scale,
                                  o=o_sparse, lse=l_sparse, ws=ws_dense)
            marks.append(("router", a, b))
            marks.append(("sparse", b, ev()))
        if args.only in ("all", "via"):
            a = ev()
            api.attn_dense_tara_via(qd, kd, vd, segd, td, seg, t, *tara, scale=scale, o=o_via,
                                    lse=l_via, ws=ws_via)
            marks.append(("via", a, ev()))
        return marks

    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        print(f"# warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    all_marks = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        all_marks.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for marks in all_marks:
        for name, a, b in marks:
            rows[name].append(a.elapsed_time(b))
    print(f"# timed {args.steps} steps in {wall:.2f}s", file=sys.stderr, flush=True)

    ms_step = wall * 1e3 / args.steps
    calls = call_summaries(rows, dense_flop, args.sparsity, k_sel, n_prot, kept)
    value = headline_value(calls)
    d = calls.get("dense_tara")

    sweep = {}
    if not args.no_sweep and args.only in ("all", "sparse"):
        for sp in wl.sparsities:
            pl = api.router_plan(seg, wl.protected_prefix_len, sp)
            tl = torch.empty((H, nb, pl["k_sel"]), dtype=torch.int32, device="cuda")
            rt, st = [], []
            for rep in range(4):
                a = ev()
                api.attn_block_router(qd, kd, segd, wl.protected_prefix_len, pl["k_sel"], n_prot,
                                      tiles=tl, prot=prot, ws=ws_router)
                b = ev()
                api.attn_block_sparse(qd, kd, vd, segd, td, tl, prot, *tara, scale=scale,
                                      o=o_sparse, lse=l_sparse, ws=ws_dense)
                c = ev()
                torch.cuda.synchronize()
                if rep:
                    rt.append(a.elapsed_time(b))
                    st.append(b.elapsed_time(c))
            kf = (n_prot + pl["k_sel"]) / nb
            tot = float(np.median(rt) + np.median(st))
            sweep[f"{sp:.2f}"] = {"k_sel": pl["k_sel"], "kept_frac": kf,
                                  "router_ms": float(np.median(rt)),
                                  "sparse_ms": float(np.median(st)),
                                  "speedup_vs_dense": (d["ms"] / tot) if d else None,
                                  "ideal_speedup": 1.0 / kf}
        print("# sweep done", file=sys.stderr, flush=True)

    # The isolated shape timed on the Flash Partitions page (107,126 rows x 8 heads): direct
    # and partition-path calls, reported beside the page's figures (another GPU: context).
    p1 = None
    if not args.no_sweep and args.only == "all":
        w1 = W.P1_MICRO
        q1, k1, v1 = (dev(x) for x in W.make_qkv(w1))
        s1, t1 = W.layout(w1)
        s1d, t1d = torch.from_numpy(s1).cuda(), torch.from_numpy(t1).cuda()
        o1 = torch.empty_like(q1)
        l1 = torch.empty((w1.n, w1.heads), dtype=torch.float32, device="cuda")
        ws1 = torch.empty(api.dense_tara_workspace_bytes(w1.n, w1.heads, w1.head_dim, 1),
                          dtype=torch.uint8, device="cuda")
        wv1 = torch.empty(api.via_workspace_bytes(s1, t1, w1.heads, w1.head_dim, 1),
                          dtype=torch.uint8, device="cuda")
        f1 = 4.0 * w1.n * w1.n * w1.head_dim * w1.heads
        p1 = {"workload": "107,126 rows x 8 heads x d 128 bf16, TARA defaults",
              "dense_equiv_tflop": f1 / 1e12,
              "page_context_s": {"native_flash_attention": 0.327, "flash_partitions": 0.422,
                                 "temporal_flex_attention": 0.628,
                                 "hardware": "RTX PRO 6000 Blackwell (another GPU)"}}
        for name, fn in (("direct", lambda: api.attn_dense_tara(
                             q1, k1, v1, s1d, t1d, s1d, t1d, *w1.tara, scale=w1.scale, o=o1,
                             lse=l1, ws=ws1)),
                         ("via", lambda: api.attn_dense_tara_via(
                             q1, k1, v1, s1d, t1d, s1, t1, *w1.tara, scale=w1.scale, o=o1,
                             lse=l1, ws=wv1))):
            ts = []
            for rep in range(4):
                a = ev()
                fn()
                b = ev()
                torch.cuda.synchronize()
                if rep:
                    ts.append(a.elapsed_time(b))
            ms1 = float(np.median(ts))
            p1[name] = {"ms": ms1, "dense_equiv_tflops": f1 / (ms1 * 1e-3) / 1e12}
        print("# isolated shape done", file=sys.stderr, flush=True)

    # NEXT row: the pooled tail term at the benchmark sparsity (router with tail + sparse with
    # tail), outside the step value
    next_rows = None
    if not args.no_sweep and args.only == "all":
        tl_lse = torch.empty((H, nb), dtype=torch.float32, device="cuda")
        tl_v = torch.empty((H, nb, D), dtype=torch.float32, device="cuda")
        ws_rt = torch.empty(api.router_tail_workspace_bytes(N, H, D), dtype=torch.uint8,
                            device="cuda")
        rt, st = [], []
        for rep in range(4):
            a = ev()
            api.attn_block_router_tail(qd, kd, vd, segd, wl.protected_prefix_len, k_sel, n_prot,
                                       scale=scale, tiles=tiles, prot=prot, tail_lse=tl_lse,
                                       tail_v=tl_v, ws=ws_rt)
            b = ev()
            api.attn_block_sparse_tail(qd, kd, vd, segd, td, tiles, prot, tl_lse, tl_v, *tara,
                                       scale=scale, o=o_sparse, lse=l_sparse, ws=ws_dense)
            c = ev()
            torch.cuda.synchronize()
            if rep:
                rt.append(a.elapsed_time(b))
                st.append(b.elapsed_time(c))
        tot = float(np.median(rt) + np.median(st))
        next_rows = {"tail_correction": {
            "sparsity": args.sparsity, "router_tail_ms": float(np.median(rt)),
            "sparse_tail_ms": float(np.median(st)), "ms": tot,
            "speedup_vs_dense": (d["ms"] / tot) if d else None}}
        print("# tail term done", file=sys.stderr, flush=True)

        # routing variants at the benchmark sparsity: blocks of 32 and 128 rows, and audio
        # sink query blocks (dense) at 64
        def time_pair(route, attend):
            rt, st = [], []
            for rep in range(4):
                a = ev()
                route()
                b = ev()
                attend()
                c = ev()
                torch.cuda.synchronize()
                if rep:
                    rt.append(a.elapsed_time(b))
                    st.append(b.elapsed_time(c))
            r_ms, s_ms = float(np.median(rt)), float(np.median(st))
            return {"router_ms": r_ms, "sparse_ms": s_ms, "ms": r_ms + s_ms,
                    "speedup_vs_dense": (d["ms"] / (r_ms + s_ms)) if d else None}

        for bsz in (32, 128):
            pv = api.router_plan(seg, wl.protected_prefix_len, args.sparsity, block_size=bsz)
            tv_, pr_ = api.attn_block_router(qd, kd, segd, wl.protected_prefix_len, pv["k_sel"],
                                             pv["n_prot"], block_size=bsz)
            ws_v = torch.empty(api.router_workspace_bytes(N, H, D, bsz), dtype=torch.uint8,
                               device="cuda")
            row = time_pair(
                lambda: api.attn_block_router(qd, kd, segd, wl.protected_prefix_len,
                                              pv["k_sel"], pv["n_prot"], block_size=bsz,
                                              tiles=tv_, prot=pr_, ws=ws_v),
                lambda: api.attn_block_sparse(qd, kd, vd, segd, td, tv_, pr_, *tara,
                                              scale=scale, block_size=bsz, o=o_sparse,
                                              lse=l_sparse, ws=ws_dense))
            row.update({"sparsity": args.sparsity, "k_sel": pv["k_sel"],
                        "kept_frac": (pv["n_prot"] + pv["k_sel"]) / pv["nb"]})
            next_rows[f"block_size_{bsz}"] = row
            del tv_, pr_, ws_v
        row = time_pair(
            lambda: api.attn_block_router(qd, kd, segd, wl.protected_prefix_len, k_sel, n_prot,
                                          tiles=tiles, prot=prot, ws=ws_router),
            lambda: api.attn_block_sparse_sinks(qd, kd, vd, segd, td, tiles, prot,
                                                1 << W.SEG_AUDIO, None, None, *tara,
                                                scale=scale, o=o_sparse, lse=l_sparse,
                                                ws=ws_dense))
        row.update({"sparsity": args.sparsity, "block_size": 64,
                    "sink_query_blocks_per_head": int(sum(
                        1 for b in range(nb)
                        if np.any(seg[b * 64:(b + 1) * 64] == W.SEG_AUDIO)))})
        next_rows["audio_sink_queries"] = row
        print("# routing variants done", file=sys.stderr, flush=True)

        # int8 QK product on the attended tiles (per-token quantization of q and k inside
        # the call), block 64, same router lists
        ws_i8 = torch.empty(api.int8qk_workspace_bytes(N, H, D), dtype=torch.uint8,
                            device="cuda")
        row = time_pair(
            lambda: api.attn_block_router(qd, kd, segd, wl.protected_prefix_len, k_sel, n_prot,
                                          tiles=tiles, prot=prot, ws=ws_router),
            lambda: api.attn_block_sparse_int8qk(qd, kd, vd, segd, td, tiles, prot, None, None,
                                                 0, *tara, scale=scale, o=o_sparse,
                                                 lse=l_sparse, ws=ws_i8))
        row.update({"sparsity": args.sparsity, "block_size": 64,
                    "note": "sparse_ms includes the int8 quantization of q and k"})
        next_rows["int8_qk"] = row
        del ws_i8
        print("# int8 QK done", file=sys.stderr, flush=True)

        # reference-protection quota on the guide span (Light: the best 15% of the guide
        # tiles on top of the ordinary top-k; Heavy: every guide tile protected)
        for mode, name in ((api.H3_REF_LIGHT, "light"), (api.H3_REF_HEAVY, "heavy")):
            pr_ = api.router_plan_ref(seg, wl.protected_prefix_len, args.sparsity, mode)
            tr_ = torch.empty((H, nb, pr_["k_sel"]), dtype=torch.int32, device="cuda")
            pp_ = torch.empty((pr_["n_prot"],), dtype=torch.int32, device="cuda")
            row = time_pair(
                lambda: api.attn_block_router_ref(qd, kd, segd, seg, wl.protected_prefix_len,
                                                  args.sparsity, mode, tiles=tr_, prot=pp_,
                                                  ws=ws_router),
                lambda: api.attn_block_sparse(qd, kd, vd, segd, td, tr_, pp_, *tara,
                                              scale=scale, o=o_sparse, lse=l_sparse,
                                              ws=ws_dense))
            row.update({"sparsity": args.sparsity, "block_size": 64, "list_width": pr_["k_sel"],
                        "n_prot": pr_["n_prot"]})
            next_rows[f"reference_protection_{name}"] = row
            del tr_, pp_
        print("# reference protection done", file=sys.stderr, flush=True)

    roofline = None
    if d:
        traffic = None
        if os.path.exists(PMC_SUMMARY):
            with open(PMC_SUMMARY) as f:
                pmc = json.load(f)
            if pmc.get("source_hash") == kernel_source_hash():
                traffic = pmc.get("hbm_bytes_per_launch")
        achieved = dense_flop / (d["ms_mean"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                    "kernel": DENSE_KERNEL,
                    "per_launch": "4*N^2*d*H = 391.71 TFLOP (116,883 x 116,883 x 128 x 56)",
                    "timing": "HIP events on the launch stream around each attn_dense_tara call "
                              "(includes the key pre-passes), mean over timed steps"}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, q, k, v, seg, t)
        print("# cpu baseline done", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "packed sequence 116,883 rows x 56 heads x d 128 bf16: dense "
                               "TARA direct + router/block-sparse s=%.2f + partition path; "
                               "value = the dense TARA call" % args.sparsity,
                   "rows": N, "heads": H, "head_dim": D, "block_size": 64,
                   "sparsity": args.sparsity, "step_rows": args.only,
                   "tara": {"strength": tara[0], "window": tara[1], "falloff": tara[2],
                            "cap": tara[3]}},
        "calls": calls,
        "sparsity_sweep": sweep,
        "isolated_shape": p1,
        "next_rows": next_rows,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
