#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Workload: one decode step of a Llama-3.1-8B-shaped attention layer at 128K
context, batch 8 (32 query heads, 8 KV heads, head_dim 128, bf16 KV in 64-token
blocks; keys a block-coherent Gaussian mixture, seeded synthetic data).

One timed step runs every stage of the hot path over that batch:
  dense   split-KV decode + merge over all 2048 blocks      (full attention)
  sparse  centroid scores + top-k (10% + sink + last 64) + listed-block decode + merge
  art     ART early-terminated decode, block 0 then most recent first (64 units,
          each streamed by 4 workgroups through a device-memory ring)
  window  sink + recent-window decode + merge                 (routed SA layer)
Optional (--stages ...,art_imp): centroid scores + importance order + ART
visiting block 0 then blocks by descending centroid score.  Optional
(--stages ...,sparse2): two-level selection (super-blocks of 16 blocks, 32
opened, then the same 205 picks + sink + window) + listed-block decode + merge.
Optional (--stages ...,dense_paged): the dense stage over a paged cache whose
blocks sit in a randomly permuted pool, addressed through a block table.
Block centroids are built once before timing (they change only when a block
fills).  Each stage reads its own copy of the KV cache so that no stage is
served from the 256 MB last-level cache filled by the previous one.

value = algorithmic HBM bytes of the step / step time (GB/s).  The roofline
object reports the dense decode kernel alone: its algorithmic bytes per launch
over its average launch time, from HIP events on the launch stream.  The CPU
baseline times the float64 oracle on a sample of (batch row, KV head) units.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
T_PROCESS = time.perf_counter()  # the whole run's wall time is reported with the line
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention HBM GB/s (% of peak) + tokens/sec at 128K ctx, batch 8"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_decode128k_b8.md")
DENSE_SOURCES = ("decode.hip", "device_common.hpp", "kernels.hpp")


def measured_dense_traffic(splits):
    """HBM bytes per dense-kernel launch from the committed counter summary,
    or None when the kernel sources changed since the counters were taken or
    the launch uses another split count."""
    import hashlib

    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if "=" in line and line.strip().startswith("dense_decode_"):
                key, val = (x.strip() for x in line.split("=", 1))
                kv[key] = val
        h = hashlib.sha256()
        for f in DENSE_SOURCES:
            with open(os.path.join(ROOT, "sparse_kv_amd", "csrc", f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != kv.get("dense_decode_source_sha256"):
            return None
        if int(kv.get("dense_decode_splits", -1)) != splits:
            return None
        return int(kv["dense_decode_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def art_groups(units):
    """Workgroups per (b, kv head) that attn_decode_art_ws launches on this device."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return min(4, cus // units) if units <= 128 and 2 * units <= cus else 1


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--splits", type=int, default=4,
                    help="splits per (batch row, KV head), dense stage (4: one workgroup per CU at batch 8)")
    ap.add_argument("--sparse-splits", type=int, default=3, help="splits per unit, sparse stage")
    ap.add_argument("--window-splits", type=int, default=3, help="splits per unit, sink+window stage")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (32K batch 8 dense, 64K batch 32 ART, the 36-layer 256K stack) "
                         "and the read-ceiling probe that the default run adds to the line")
    ap.add_argument("--stages", default="dense,sparse,art,window",
                    help="comma list of dense, sparse, art, window (the step), and art_imp, sparse2, dense_paged, "
                         "art_sel, sparse_fc, centroid_upd")
    ap.add_argument("--splits-per-shard", type=int, default=4, help="hybrid256k: inner splits per context shard")
    ap.add_argument("--sa-splits", type=int, default=32, help="hybrid256k: splits of a sink+window layer")
    ap.add_argument("--workload", default="decode128k", choices=["decode128k", "art64k", "hybrid256k", "dense32k"],
                    help="decode128k (default): the 128K batch-8 step above; art64k: ART on the 64K batch-32 "
                         "recency workload vs dense; hybrid256k: 36-layer routed stack at 256K vs all-full; "
                         "dense32k: dense split-KV decode + merge at 32K batch 8 (needle keys)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the decode path is single-device; across GPUs it would shard by (batch row, KV head) units, or by "
              "sequence ranges whose states attn_merge_states combines).", file=sys.stderr)
        sys.exit(2)

    if args.workload == "art64k":
        return bench_art64k(args)
    if args.workload == "hybrid256k":
        return bench_hybrid256k(args)
    if args.workload == "dense32k":
        return bench_dense32k(args)

    import numpy as np
    import torch

    import sparse_kv_amd as skv
    import synth

    stages = [s for s in args.stages.split(",") if s]
    W = synth.WORKLOADS[3]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    NB = L // 64
    topk, n_sink, n_recent = W["topk"], W["n_sink"], W["n_recent"]
    win_recent = 128
    tau, phi, patience, probe = 1e-3, 1e-4, 2, 8
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    # the read ceiling is probed first, on a fresh 4 GiB buffer, before anything else is allocated
    ceil = None if args.no_extra else run_ceiling()
    t0 = time.perf_counter()
    inp = synth.workload_inputs(3)  # units whose decisions would sit inside the margins are redrawn
    gen_s = time.perf_counter() - t0
    print(f"[bench] generated 128K batch-8 inputs in {gen_s:.1f}s", file=sys.stderr, flush=True)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    q = up(inp.q)
    copies = {}
    k0, v0 = up(inp.k), up(inp.v)
    for i, s in enumerate(("dense", "sparse", "art", "window", "art_imp", "sparse2", "art_sel", "sparse_fc",
                           "centroid_upd")):
        if s in stages or s == "dense":
            copies[s] = (k0, v0) if i == 0 else (k0.clone(), v0.clone())
    torch.cuda.synchronize()

    # prefill-time work: centroids of the sparse stage's cache, the window list
    c_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    c_ev[0].record()
    C = skv.attn_build_centroids(copies["sparse"][0]) if "sparse" in stages else None
    c_ev[1].record()
    C_imp = skv.attn_build_centroids(copies["art_imp"][0]) if "art_imp" in stages else None
    if "dense_paged" in stages:
        # pool[perm[i]] = logical block i (row-major over (b, j)); table[b, j] = perm[b * NB + j]
        perm = torch.randperm(B * NB, generator=torch.Generator().manual_seed(5), dtype=torch.int64).to(dev)

        def to_pool(x):
            blocks = x.view(B, Hkv, NB, 64, d).permute(0, 2, 1, 3, 4).reshape(B * NB, Hkv, 64, d)
            pool = torch.empty_like(blocks)
            pool[perm] = blocks
            return pool

        kpool, vpool = to_pool(k0), to_pool(v0)
        ptable = perm.view(B, NB).to(torch.int32).contiguous()
    # ART over the top-k selection; selection by a per-KV-head forecast vector; the per-step centroid refresh
    C_sel = skv.attn_build_centroids(copies["art_sel"][0]) if "art_sel" in stages else None
    C_fc = skv.attn_build_centroids(copies["sparse_fc"][0]) if "sparse_fc" in stages else None
    C_up = skv.attn_build_centroids(copies["centroid_upd"][0]) if "centroid_upd" in stages else None
    fcq = torch.randn((B, Hkv, d), generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(dev)
    prev_lens = torch.full((B,), L - 1, dtype=torch.int32, device=dev)  # one token appended per row
    group2, kc2 = 16, 32
    C_2 = skv.attn_build_centroids(copies["sparse2"][0]) if "sparse2" in stages else None
    C2_2 = skv.attn_build_super_centroids(C_2, group2) if "sparse2" in stages else None
    win_idx, win_n = skv.attn_select_topk(None, None, k=0, n_sink_blocks=n_sink, n_recent_blocks=win_recent,
                                          shape=(B, Hkv, NB), device=dev)
    torch.cuda.synchronize()
    centroid_ms = c_ev[0].elapsed_time(c_ev[1])

    f32 = dict(dtype=torch.float32, device=dev)
    S, Ss, Sw = args.splits, args.sparse_splits, args.window_splits
    st_d = (torch.empty((B, Hq, S), **f32), torch.empty((B, Hq, S), **f32), torch.empty((B, Hq, S, d), **f32))
    st_s = (torch.empty((B, Hq, Ss), **f32), torch.empty((B, Hq, Ss), **f32), torch.empty((B, Hq, Ss, d), **f32))
    st_w = (torch.empty((B, Hq, Sw), **f32), torch.empty((B, Hq, Sw), **f32), torch.empty((B, Hq, Sw, d), **f32))
    out_d, out_s, out_w, out_a = (torch.empty((B, Hq, d), **f32) for _ in range(4))
    st_p = (torch.empty((B, Hq, S), **f32), torch.empty((B, Hq, S), **f32), torch.empty((B, Hq, S, d), **f32))
    out_p = torch.empty((B, Hq, d), **f32)
    scores = torch.empty((B, Hkv, NB), **f32)
    max_sel = n_sink + n_recent + topk
    sel_idx = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    sel_n = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    stop = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    fetched = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    scores_i = torch.empty((B, Hkv, NB), **f32)
    sel2_idx = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    sel2_n = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    st_2 = (torch.empty((B, Hq, Ss), **f32), torch.empty((B, Hq, Ss), **f32), torch.empty((B, Hq, Ss, d), **f32))
    out_2 = torch.empty((B, Hq, d), **f32)
    order_i = torch.empty((B, Hkv, NB), dtype=torch.int32, device=dev)
    # ART spreads each (b, kv head) over several CUs through this workspace when B * Hkv is small
    art_ws = torch.empty(max(skv.attn_art_workspace_bytes(q, k0), 1), dtype=torch.uint8, device=dev)
    out_i = torch.empty((B, Hq, d), **f32)
    scores_a, scores_f = torch.empty((B, Hkv, NB), **f32), torch.empty((B, Hkv, NB), **f32)
    sela_idx = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    sela_n = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    self_idx = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    self_n = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    out_as, out_f = torch.empty((B, Hq, d), **f32), torch.empty((B, Hq, d), **f32)
    stop_as = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    fetched_as = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    st_f = (torch.empty((B, Hq, Ss), **f32), torch.empty((B, Hq, Ss), **f32), torch.empty((B, Hq, Ss, d), **f32))
    stop_i = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    fetched_i = torch.empty((B, Hkv), dtype=torch.int32, device=dev)

    names = ["dense_kernel", "dense_merge", "sparse", "art", "window"]
    ev = {}

    ev_timed = {}
    # events are created before the passes that record them, so that recording
    # adds no host work that could let the device run dry between stages
    ev_pool = [torch.cuda.Event(enable_timing=True) for _ in range(32 * args.steps)]

    def step(record):
        # record: "all" (every stage boundary, into ev), "dense" (the dense
        # kernel's two boundaries only, into ev_timed) or None
        def mark(tag):
            if record == "all" or (record == "dense" and tag.startswith("dense_kernel")):
                e = ev_pool.pop() if ev_pool else torch.cuda.Event(enable_timing=True)
                e.record()
                (ev if record == "all" else ev_timed).setdefault(tag, []).append(e)

        if "dense" in stages:
            kd, vd = copies["dense"]
            mark("dense_kernel.0")
            skv.attn_decode_dense(q, kd, vd, None, num_splits=S, m=st_d[0], l=st_d[1], o=st_d[2])
            mark("dense_kernel.1")
            skv.attn_merge_states(*st_d, out=out_d)
            mark("dense_merge.1")
        if "sparse" in stages:
            ks, vs = copies["sparse"]
            mark("sparse.0")
            skv.attn_score_centroids(q, C, None, out=scores)
            skv.attn_select_topk(scores, None, k=topk, n_sink_blocks=n_sink, n_recent_blocks=n_recent,
                                 max_sel=max_sel, block_idx=sel_idx, n_sel=sel_n)
            skv.attn_decode_sparse(q, ks, vs, sel_idx, sel_n, None, num_splits=Ss, m=st_s[0], l=st_s[1], o=st_s[2])
            skv.attn_merge_states(*st_s, out=out_s)
            mark("sparse.1")
        if "art" in stages:
            ka, va = copies["art"]
            mark("art.0")
            skv.attn_decode_art_ws(q, ka, va, None, tau=tau, phi=phi, patience=patience, probe_dim=probe,
                                   workspace=art_ws, out=out_a, stop_pos=stop, blocks_fetched=fetched)
            mark("art.1")
        if "window" in stages:
            kw, vw = copies["window"]
            mark("window.0")
            skv.attn_decode_sparse(q, kw, vw, win_idx, win_n, None, num_splits=Sw, m=st_w[0], l=st_w[1], o=st_w[2])
            skv.attn_merge_states(*st_w, out=out_w)
            mark("window.1")
        if "dense_paged" in stages:
            mark("dense_paged.0")
            skv.attn_decode_dense_paged(q, kpool, vpool, ptable, None, num_splits=S, m=st_p[0], l=st_p[1], o=st_p[2])
            mark("dense_paged.k")
            skv.attn_merge_states(*st_p, out=out_p)
            mark("dense_paged.1")
        if "sparse2" in stages:
            k2, v2 = copies["sparse2"]
            mark("sparse2.0")
            skv.attn_select_two_level(q, C_2, C2_2, group2, None, k_coarse=kc2, k=topk, n_sink_blocks=n_sink,
                                      n_recent_blocks=n_recent, max_sel=max_sel, block_idx=sel2_idx, n_sel=sel2_n)
            mark("sparse2.sel")
            skv.attn_decode_sparse(q, k2, v2, sel2_idx, sel2_n, None, num_splits=Ss, m=st_2[0], l=st_2[1], o=st_2[2])
            skv.attn_merge_states(*st_2, out=out_2)
            mark("sparse2.1")
        if "art_imp" in stages:
            ki, vi = copies["art_imp"]
            mark("art_imp.0")
            skv.attn_score_centroids(q, C_imp, None, out=scores_i)
            mark("art_imp.score")
            skv.attn_order_blocks(scores_i, None, out=order_i)
            mark("art_imp.order")
            skv.attn_decode_art_ws(q, ki, vi, None, order=order_i, tau=tau, phi=phi, patience=patience,
                                   probe_dim=probe, workspace=art_ws, out=out_i, stop_pos=stop_i,
                                   blocks_fetched=fetched_i)
            mark("art_imp.1")
        if "art_sel" in stages:
            ka, va = copies["art_sel"]
            mark("art_sel.0")
            skv.attn_score_centroids(q, C_sel, None, out=scores_a)
            skv.attn_select_topk(scores_a, None, k=topk, n_sink_blocks=n_sink, n_recent_blocks=n_recent,
                                 max_sel=max_sel, block_idx=sela_idx, n_sel=sela_n)
            mark("art_sel.sel")
            skv.attn_decode_art_list_ws(q, ka, va, sela_idx, sela_n, None, tau=tau, phi=phi, patience=patience,
                                        probe_dim=probe, workspace=art_ws, out=out_as, stop_pos=stop_as,
                                        blocks_fetched=fetched_as)
            mark("art_sel.1")
        if "sparse_fc" in stages:
            kf_, vf_ = copies["sparse_fc"]
            mark("sparse_fc.0")
            skv.attn_score_centroids(fcq, C_fc, None, scale=d ** -0.5, out=scores_f)
            skv.attn_select_topk(scores_f, None, k=topk, n_sink_blocks=n_sink, n_recent_blocks=n_recent,
                                 max_sel=max_sel, block_idx=self_idx, n_sel=self_n)
            skv.attn_decode_sparse(q, kf_, vf_, self_idx, self_n, None, num_splits=Ss, m=st_f[0], l=st_f[1], o=st_f[2])
            skv.attn_merge_states(*st_f, out=out_f)
            mark("sparse_fc.1")
        if "centroid_upd" in stages:
            mark("centroid_upd.0")
            skv.attn_update_centroids(copies["centroid_upd"][0], C_up, None, prev_lens=prev_lens, span_hint=1)
            mark("centroid_upd.1")

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    # the timed steps carry only the two events around the dense kernel (its
    # launch duration for the roofline, on the stream it runs on); a second
    # pass of the same steps records every stage boundary for the breakdown
    # (a stage-boundary event costs a few microseconds)
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step("dense")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    for _ in range(args.steps):
        step("all")
    torch.cuda.synchronize()
    # detector overhead of both ART launch forms on this input: tau = phi = 0 (no stop, every probe
    # compared) against the detector off; every block of every unit is folded either way
    art_overhead = {}
    if "art" in stages:
        ka, va = copies["art"]
        o_, s_, f_ = torch.empty_like(out_a), torch.empty_like(stop), torch.empty_like(fetched)
        art_overhead["across_workgroups"] = detector_overhead(
            lambda **kw: skv.attn_decode_art_ws(q, ka, va, None, workspace=art_ws, out=o_, stop_pos=s_,
                                                blocks_fetched=f_, **kw), patience)
        art_overhead["one_workgroup"] = detector_overhead(
            lambda **kw: skv.attn_decode_art(q, ka, va, None, out=o_, stop_pos=s_, blocks_fetched=f_, **kw),
            patience, reps=3)

    def avg_ms(a, b, evs=None):
        evs = ev if evs is None else evs
        xs = [e0.elapsed_time(e1) for e0, e1 in zip(evs[a], evs[b])]
        return sum(xs) / len(xs)

    # algorithmic bytes per stage
    kv_block = 64 * d * 2 * 2  # K + V bytes of one block of one KV head
    q_bytes = B * Hq * d * 2
    o_bytes = B * Hq * d * 4
    units = B * Hkv
    paths = {}
    total_bytes = 0.0
    gbs = lambda by, ms: by / (ms * 1e-3) / 1e9
    if "dense" in stages:
        kern_ms = avg_ms("dense_kernel.0", "dense_kernel.1", ev_timed)  # inside the timed steps
        path_ms = avg_ms("dense_kernel.0", "dense_merge.1")
        by = units * NB * kv_block + q_bytes + o_bytes
        total_bytes += by
        paths["dense"] = dict(ms=path_ms, kernel_ms=kern_ms, bytes=by, gbs=gbs(by, path_ms),
                              pct_peak=100 * gbs(by, path_ms) / PEAK_HBM_GBS, tokens_per_s=B / (path_ms * 1e-3),
                              splits=S)
    if "sparse" in stages:
        n_sel = sel_n.cpu().numpy()
        ms = avg_ms("sparse.0", "sparse.1")
        by = float(n_sel.sum()) * kv_block + units * NB * d * 4 + units * NB * 4 * 2 + q_bytes + o_bytes
        total_bytes += by
        paths["sparse"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), blocks_per_unit=float(n_sel.mean()),
                               tokens_per_s=B / (ms * 1e-3), splits=Ss)
    if "art" in stages:
        st = unit_stats(stop.cpu().numpy(), fetched.cpu().numpy(), Hkv)
        ms = avg_ms("art.0", "art.1")
        by = st["blocks_needed_per_unit"] * units * kv_block + q_bytes + o_bytes
        total_bytes += by
        paths["art"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), tokens_per_s=B / (ms * 1e-3),
                            workgroups_per_unit=art_groups(B * Hkv), **st,
                            detector_overhead_pct=art_overhead)
    if "window" in stages:
        ms = avg_ms("window.0", "window.1")
        by = float(win_n.cpu().numpy().sum()) * kv_block + q_bytes + o_bytes
        total_bytes += by
        paths["window"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), tokens_per_s=B / (ms * 1e-3), splits=Sw)
    if "dense_paged" in stages:
        ms = avg_ms("dense_paged.0", "dense_paged.1")
        by = units * NB * kv_block + q_bytes + o_bytes + B * NB * 4
        total_bytes += by
        paths["dense_paged"] = dict(ms=ms, kernel_ms=avg_ms("dense_paged.0", "dense_paged.k"), bytes=by,
                                    gbs=gbs(by, ms), tokens_per_s=B / (ms * 1e-3), splits=S)
        if "dense" in stages:
            paths["dense_paged"]["max_abs_diff_vs_contiguous"] = float((out_p - out_d).abs().max())
    if "sparse2" in stages:
        n2 = sel2_n.cpu().numpy()
        ms = avg_ms("sparse2.0", "sparse2.1")
        NS2 = -(-NB // group2)
        by = (float(n2.sum()) * kv_block + units * NS2 * d * 4 + units * kc2 * group2 * d * 4 + q_bytes + o_bytes)
        total_bytes += by
        paths["sparse2"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), select_ms=avg_ms("sparse2.0", "sparse2.sel"),
                                blocks_per_unit=float(n2.mean()), group=group2, opened=kc2,
                                tokens_per_s=B / (ms * 1e-3), splits=Ss)
        if "dense" in stages:
            paths["sparse2"]["max_abs_err_vs_dense"] = float((out_2.double() - out_d.double()).abs().max())
            if "sparse" in stages:
                paths["sparse"]["max_abs_err_vs_dense"] = float((out_s.double() - out_d.double()).abs().max())
    if "art_imp" in stages:
        stp = stop_i.cpu().numpy().reshape(B, Hkv, Hq // Hkv)
        need = stp.max(axis=2) + 1
        ms = avg_ms("art_imp.0", "art_imp.1")
        by = (float(need.sum()) * kv_block + units * NB * d * 4 + units * NB * 4 * 2 + units * NB * 4
              + float(need.sum()) * 4 + q_bytes + o_bytes)
        total_bytes += by
        paths["art_imp"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), score_ms=avg_ms("art_imp.0", "art_imp.score"),
                                order_ms=avg_ms("art_imp.score", "art_imp.order"),
                                art_ms=avg_ms("art_imp.order", "art_imp.1"), mean_stop=float(stp.mean()),
                                blocks_needed_per_unit=float(need.mean()),
                                blocks_fetched_per_unit=float(fetched_i.cpu().numpy().mean()),
                                tokens_per_s=B / (ms * 1e-3))
        if "dense" in stages:
            # accuracy against full attention, recency-first and importance-first
            ref = out_d.double()
            paths["art_imp"]["max_abs_err_vs_dense"] = float((out_i.double() - ref).abs().max())
            if "art" in stages:
                paths["art"]["max_abs_err_vs_dense"] = float((out_a.double() - ref).abs().max())
    if "art_sel" in stages:
        stp = stop_as.cpu().numpy().reshape(B, Hkv, Hq // Hkv)
        need = stp.max(axis=2) + 1
        ms = avg_ms("art_sel.0", "art_sel.1")
        by = (float(need.sum()) * kv_block + units * NB * d * 4 + units * NB * 4 * 2 + float(need.sum()) * 4
              + q_bytes + o_bytes)
        total_bytes += by
        paths["art_sel"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), select_ms=avg_ms("art_sel.0", "art_sel.sel"),
                                art_ms=avg_ms("art_sel.sel", "art_sel.1"), mean_stop=float(stp.mean()),
                                listed_per_unit=float(sela_n.cpu().numpy().mean()),
                                blocks_needed_per_unit=float(need.mean()),
                                blocks_fetched_per_unit=float(fetched_as.cpu().numpy().mean()),
                                tokens_per_s=B / (ms * 1e-3))
    if "sparse_fc" in stages:
        nf = self_n.cpu().numpy()
        ms = avg_ms("sparse_fc.0", "sparse_fc.1")
        by = float(nf.sum()) * kv_block + units * NB * d * 4 + units * NB * 4 * 2 + q_bytes + o_bytes
        total_bytes += by
        paths["sparse_fc"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), blocks_per_unit=float(nf.mean()),
                                  tokens_per_s=B / (ms * 1e-3), splits=Ss)
    if "centroid_upd" in stages:
        ms = avg_ms("centroid_upd.0", "centroid_upd.1")
        by = units * (kv_block // 2) + units * d * 4  # the last block's K read, its centroid written
        total_bytes += by
        paths["centroid_upd"] = dict(ms=ms, bytes=by, gbs=gbs(by, ms), blocks_per_unit=1)
    if "dense" in paths:
        for k_ in ("sparse", "art", "window", "art_imp", "sparse2", "dense_paged", "art_sel", "sparse_fc"):
            if k_ in paths:
                paths[k_]["speedup_vs_dense"] = paths["dense"]["ms"] / paths[k_]["ms"]

    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode step, 128K context, batch 8, 32 q / 8 kv heads, d 128, bf16 KV, "
                               "64-token blocks; dense + centroid top-k sparse + ART + sink/window stages",
                   "batch": B, "context": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "block": 64,
                   "stages": stages, "parallelism": "single-gpu"},
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(paths["dense"]["tokens_per_s"], 1) if "dense" in paths else None,
        "centroid_build_ms": round(centroid_ms, 4),
        "paths": {k_: rounded(v_) for k_, v_ in paths.items()},
    }
    if "dense" in paths:
        kb = units * NB * kv_block + q_bytes + B * Hq * S * (d + 2) * 4
        ach = kb / (paths["dense"]["kernel_ms"] * 1e-3) / 1e9
        res["roofline"] = {"kernel": "decode_kernel (split-KV dense)", "bound": "hbm", "achieved": round(ach, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                           "traffic": measured_dense_traffic(S), "bytes_per_launch": kb,
                           "avg_launch_ms": round(paths["dense"]["kernel_ms"], 5)}
    if not args.no_extra:
        # the other workloads, each on its own inputs; the line's metric stays the 128K step
        del copies
        torch.cuda.empty_cache()
        res["ceiling"] = rounded(ceil)
        if "roofline" in res:
            res["roofline"]["ceiling_gbs"] = round(ceil["gbs"], 1)
            res["roofline"]["frac_of_ceiling"] = round(res["roofline"]["achieved"] / ceil["gbs"], 4)
        if "dense" in res["paths"]:
            res["paths"]["dense"]["pct_of_ceiling"] = round(100 * paths["dense"]["gbs"] / ceil["gbs"], 2)
        for name, fn in (("dense32k_b8", run_dense32k), ("art64k_b32", run_art64k),
                         ("routed256k_36layers", run_hybrid256k)):
            t = time.perf_counter()
            r = fn(args)
            r["pct_of_ceiling"] = 100 * r["gbs"] / ceil["gbs"]
            res["paths"][name] = rounded(r)
            print(f"[bench] {name}: {r['ms']:.4f} ms ({time.perf_counter() - t:.1f}s)", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, topk, n_sink, n_recent, win_recent,
                                           tau, phi, patience, probe, total_bytes / units)
    # every workload above ran in this one process: its wall time, against a 600 s run limit
    res["run_s"] = round(time.perf_counter() - T_PROCESS, 1)
    res["within_600s"] = res["run_s"] < 600
    print(json.dumps(res), flush=True)


def rounded(d):
    return {k_: (round(v_, 4) if isinstance(v_, float) else (rounded(v_) if isinstance(v_, dict) else v_))
            for k_, v_ in d.items()}


def _timer():
    import torch

    class T:
        def __init__(self):
            self.ev = []

        def __enter__(self):
            self.a = torch.cuda.Event(enable_timing=True)
            self.b = torch.cuda.Event(enable_timing=True)
            self.a.record()
            return self

        def __exit__(self, *exc):
            self.b.record()
            self.ev.append((self.a, self.b))

        def avg_ms(self):
            torch.cuda.synchronize()
            return sum(a.elapsed_time(b) for a, b in self.ev) / len(self.ev)

        def median_ms(self):
            torch.cuda.synchronize()
            xs = sorted(a.elapsed_time(b) for a, b in self.ev)
            return xs[len(xs) // 2]

    return T()


def _line(args, metric, value, unit, ms, config, **extra):
    res = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config}
    res.update(extra)
    print(json.dumps(res), flush=True)


def run_dense32k(args):
    """Dense split-KV decode + merge at 32K context, batch 8 (Llama-3.1-8B layer shape, needle keys)."""
    import numpy as np
    import torch

    import sparse_kv_amd as skv
    import synth

    W = synth.WORKLOADS[2]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    dev = torch.device("cuda", 0)
    inp = synth.make_inputs(2, B, Hq, Hkv, d, L, kind=W["kind"])
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    del inp
    S = args.splits
    m, l, o = skv.attn_decode_dense(q, k, v, None, num_splits=S)
    out = skv.attn_merge_states(m, l, o)
    tk, ts = _timer(), _timer()
    for i in range(args.warmup + args.steps):
        rec = i >= args.warmup
        with (ts if rec else _timer()):
            with (tk if rec else _timer()):
                skv.attn_decode_dense(q, k, v, None, num_splits=S, m=m, l=l, o=o)
            skv.attn_merge_states(m, l, o, out=out)
    NB = L // 64
    kv_bytes = B * Hkv * NB * 64 * d * 2 * 2
    by = kv_bytes + B * Hq * d * 2 + B * Hq * d * 4
    kb = kv_bytes + B * Hq * d * 2 + B * Hq * S * (d + 2) * 4
    ms, kms = ts.avg_ms(), tk.avg_ms()
    del q, k, v
    torch.cuda.empty_cache()
    return dict(workload="dense split-KV decode + merge, 32K context, batch 8, 32 q / 8 kv heads, d 128, bf16 KV, "
                         "needle keys", batch=B, context=L, splits=S, ms=ms, bytes=by, gbs=by / (ms * 1e-3) / 1e9,
                pct_peak=100 * by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, tokens_per_s=B / (ms * 1e-3), kernel_ms=kms,
                kernel_gbs=kb / (kms * 1e-3) / 1e9)


def bench_dense32k(args):
    r = run_dense32k(args)
    _line(args, "dense decode attention HBM GB/s, 32K ctx, batch 8", r["gbs"], "GB/s", r["ms"],
          {"workload": r["workload"], "batch": r["batch"], "context": r["context"], "splits": r["splits"],
           "parallelism": "single-gpu"},
          tokens_per_s=round(r["tokens_per_s"], 1), kernel_ms=round(r["kernel_ms"], 5),
          kernel_gbs=round(r["kernel_gbs"], 1), pct_of_peak_hbm=round(r["pct_peak"], 2))


def unit_stats(stop, fetched, Hkv):
    """Per (batch row, KV head) unit: blocks needed (the last head's stop + 1) and fetched."""
    import numpy as np

    B, Hq = stop.shape
    need = stop.reshape(B, Hkv, Hq // Hkv).max(axis=2) + 1
    fetched = np.asarray(fetched)
    return dict(mean_stop=float(stop.mean()), blocks_needed_per_unit=float(need.mean()),
                blocks_fetched_per_unit=float(fetched.mean()),
                needed_per_unit_min_median_p90_max=[int(need.min()), float(np.median(need)),
                                                     float(np.percentile(need, 90)), int(need.max())],
                slowest_unit_needed=int(need.max()), slowest_unit_fetched=int(fetched.flat[int(np.argmax(need))]),
                fetched_over_needed=float(fetched.sum() / need.sum()))


def run_art64k(args):
    """ART on the 64K-context batch-32 recency workload (one workgroup per (b, kv head): 256 units), dense
    on the same cache, and the detector overhead of that form (tau = phi = 0 against the detector off)."""
    import numpy as np
    import torch

    import sparse_kv_amd as skv
    import synth

    W = synth.WORKLOADS[4]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    dev = torch.device("cuda", 0)
    inp = synth.workload_inputs(4)
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    del inp
    art = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])
    out, stop, fetched = skv.attn_decode_art(q, k, v, None, **art)
    S = max(1, 256 // (B * Hkv))  # one workgroup per CU
    m, l, o = skv.attn_decode_dense(q, k, v, None, num_splits=S)
    od = skv.attn_merge_states(m, l, o)
    ta, td = _timer(), _timer()
    for i in range(args.warmup + args.steps):
        rec = i >= args.warmup
        with (ta if rec else _timer()):
            skv.attn_decode_art(q, k, v, None, out=out, stop_pos=stop, blocks_fetched=fetched, **art)
        with (td if rec else _timer()):
            skv.attn_decode_dense(q, k, v, None, num_splits=S, m=m, l=l, o=o)
            skv.attn_merge_states(m, l, o, out=od)
    over = detector_overhead(lambda **kw: skv.attn_decode_art(q, k, v, None, out=out, stop_pos=stop,
                                                              blocks_fetched=fetched, **kw), W["patience"])
    skv.attn_decode_art(q, k, v, None, out=out, stop_pos=stop, blocks_fetched=fetched, **art)
    ms_a, ms_d = ta.avg_ms(), td.avg_ms()
    st = unit_stats(stop.cpu().numpy(), fetched.cpu().numpy(), Hkv)
    kv_block = 64 * d * 4
    by = st["blocks_needed_per_unit"] * B * Hkv * kv_block + B * Hq * d * 6
    by_d = B * Hkv * (L // 64) * kv_block + B * Hq * d * 6
    del q, k, v
    torch.cuda.empty_cache()
    return dict(workload="ART decode step, 64K context, batch 32, 32 q / 8 kv heads, d 128, bf16 KV, recency-"
                         "concentrated keys; tau 1e-3, phi 1e-4, patience 2, probe 8; one workgroup per unit",
                batch=B, context=L, ms=ms_a, bytes=by, gbs=by / (ms_a * 1e-3) / 1e9, tokens_per_s=B / (ms_a * 1e-3),
                dense_ms=ms_d, dense_gbs=by_d / (ms_d * 1e-3) / 1e9, speedup_vs_dense=ms_d / ms_a,
                detector_overhead_pct=over, **st)


def detector_overhead(call, patience, reps=5):
    """Percent kernel time of the stop rule when it never fires: tau = phi = 0 (every block folded,
    every probe compared) against probe_dim = 0 (detector off); the median of interleaved runs."""
    t_on, t_off = _timer(), _timer()
    for _ in range(reps):
        with t_on:
            call(tau=0.0, phi=0.0, patience=patience, probe_dim=8)
        with t_off:
            call(tau=0.0, phi=0.0, patience=patience, probe_dim=0)
    return 100.0 * (t_on.median_ms() / t_off.median_ms() - 1.0)


def bench_art64k(args):
    r = run_art64k(args)
    extra = {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in r.items()
             if k_ not in ("workload", "batch", "context", "ms", "gbs")}
    _line(args, "ART decode attention effective HBM GB/s (needed blocks / time), 64K ctx, batch 32", r["gbs"],
          "GB/s", r["ms"], {"workload": r["workload"], "batch": r["batch"], "context": r["context"],
                            "parallelism": "single-gpu"}, **extra)


def run_hybrid256k(args):
    """One decode step of the 36-layer routed stack at 256K context, batch 1, against all-full."""
    import numpy as np
    import torch

    import sparse_kv_amd as skv
    import synth

    W = synth.WORKLOADS[5]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    nb = L // 64
    dev = torch.device("cuda", 0)
    mask = synth.route_mask(W["n_layers"], W["n_full"])
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    qs, ks, vs = [], [], []
    t0 = time.perf_counter()
    for i in range(W["n_layers"]):
        inp = synth.make_inputs(5, B, Hq, Hkv, d, L, kind="needles", layer=i)
        qs.append(up(inp.q))
        ks.append(up(inp.k))
        vs.append(up(inp.v))
        del inp
    print(f"[bench] generated 36 layers in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    sa_idx, sa_n = skv.attn_select_topk(None, None, k=0, n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"],
                                        shape=(B, Hkv, nb), device=dev)
    sps, sas = args.splits_per_shard, args.sa_splits
    kw = dict(n_shards=W["n_shards"], splits_per_shard=sps, sa_block_idx=sa_idx, sa_n_sel=sa_n, sa_splits=sas)
    ws = torch.empty(skv.attn_routed_workspace_bytes(qs[0], ks[0], W["n_shards"], sps, sas), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in qs]
    th, tf = _timer(), _timer()
    full = np.ones_like(mask)
    for i in range(args.warmup + args.steps):
        rec = i >= args.warmup
        with (th if rec else _timer()):
            skv.attn_decode_routed(qs, ks, vs, mask, None, workspace=ws, outs=outs, **kw)
        with (tf if rec else _timer()):
            skv.attn_decode_routed(qs, ks, vs, full, None, workspace=ws, outs=outs, **kw)
    ms_h, ms_f = th.avg_ms(), tf.avg_ms()
    kv_block = 64 * d * 4
    n_sa = float(sa_n.sum().item())
    by = sum((B * Hkv * nb if m_ else n_sa) * kv_block for m_ in mask) + len(mask) * B * Hq * d * 6
    by_f = len(mask) * B * Hkv * nb * kv_block + len(mask) * B * Hq * d * 6
    del qs, ks, vs, outs
    torch.cuda.empty_cache()
    return dict(workload="one decode step through a 36-layer routed stack (18 full / 18 sink+window), 256K context, "
                         f"batch 1, 32 q / 8 kv heads, d 128, bf16 KV; full layers as 8 context shards x {sps} splits",
                batch=B, context=L, splits_per_shard=sps, sa_splits=sas, ms=ms_h, bytes=by,
                gbs=by / (ms_h * 1e-3) / 1e9, pct_peak=100 * by / (ms_h * 1e-3) / 1e9 / PEAK_HBM_GBS,
                tokens_per_s=B / (ms_h * 1e-3), all_full_ms=ms_f, all_full_gbs=by_f / (ms_f * 1e-3) / 1e9,
                speedup_vs_all_full=ms_f / ms_h, byte_ratio=by_f / by)


def bench_hybrid256k(args):
    r = run_hybrid256k(args)
    _line(args, "routed hybrid decode HBM GB/s, 36 layers, 256K ctx, batch 1", r["gbs"], "GB/s", r["ms"],
          {"workload": r["workload"], "batch": r["batch"], "context": r["context"],
           "splits_per_shard": r["splits_per_shard"], "sa_splits": r["sa_splits"], "parallelism": "single-gpu"},
          tokens_per_s=round(r["tokens_per_s"], 2), all_full_ms=round(r["all_full_ms"], 4),
          all_full_gbs=round(r["all_full_gbs"], 1), speedup_vs_all_full=round(r["speedup_vs_all_full"], 3),
          byte_ratio=round(r["byte_ratio"], 3))


def run_ceiling(reps=10):
    """The achievable HBM read rate: the streaming-read probe (libsparse_kv_bench.so) over a fresh 4 GiB
    buffer, for a few grid sizes; the best median."""
    import ctypes

    import torch

    from sparse_kv_amd import build

    lib = ctypes.CDLL(build.BENCH_LIB)
    f = lib.skv_bench_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    nbytes = 4 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(2048 * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sweep = {}
    for wgs in (1024, 2048, 4096):
        t = _timer()
        for i in range(reps + 2):
            with (t if i >= 2 else _timer()):
                rc = f(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs, ctypes.c_void_p(sink.data_ptr()), stream)
                if rc != 0:
                    raise RuntimeError(f"skv_bench_stream_read failed ({rc})")
        sweep[wgs] = nbytes / (t.median_ms() * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    best = max(sweep, key=sweep.get)
    return dict(kernel="stream_read_kernel (non-temporal 16-byte loads, whole lines)", bytes=nbytes,
                gbs=sweep[best], pct_peak=100 * sweep[best] / PEAK_HBM_GBS, workgroups=best,
                sweep_gbs={str(k_): round(v_, 1) for k_, v_ in sweep.items()},
                launch_us=run_launch_floor(lib, sink, "skv_bench_empty"),
                launch_with_stores_us=run_launch_floor(lib, sink, "skv_bench_store"))


def run_launch_floor(lib, sink, probe, launches=200, reps=10):
    """Fixed cost per kernel launch: a chain of 256-workgroup launches of a probe kernel (empty, or one store
    per thread) captured in a HIP graph, replayed and timed with events; the median time per launch, in
    microseconds."""
    import ctypes

    import torch

    f = getattr(lib, probe)
    f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int

    def chain():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(launches):
            if f(256, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
                raise RuntimeError(f"{probe} failed")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    t = _timer()
    for i in range(reps + 2):
        with (t if i >= 2 else _timer()):
            g.replay()
    del g
    return t.median_ms() * 1e3 / launches


def cpu_baseline(inp, budget_s, topk, n_sink, n_recent, win_recent, tau, phi, patience, probe, bytes_per_unit):
    """Time the float64 oracle on whole (batch row, KV head) units of the same input (every stage), with
    numpy's BLAS threads as the process has them and with one thread; plus the small fp32 4K workload and
    the 32K batch-8 dense workload, each with one thread and all threads."""
    import numpy as np

    import oracle
    import synth
    from oracle.selection import forced_blocks

    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        import contextlib

        cores, threadpool_limits = 1, lambda limits: contextlib.nullcontext()
    B, Hq, Hkv, d, L = inp.shape
    G = Hq // Hkv

    def step_unit(u):
        b, g = divmod(u, Hkv)
        qf = inp.upcast(inp.q[b:b + 1, g * G:(g + 1) * G])
        kf = inp.upcast(inp.k[b:b + 1, g:g + 1])
        vf = inp.upcast(inp.v[b:b + 1, g:g + 1])
        seq = inp.seq_lens[b:b + 1]
        oracle.decode_dense(qf, kf, vf, seq, inp.scale)
        sig = oracle.centroid_scores(qf, oracle.block_centroids(kf, seq), seq, inp.scale)
        lists = oracle.select_all(sig, seq, topk, n_sink, n_recent)
        oracle.decode_blocks(qf, kf, vf, seq, inp.scale, lists)
        oracle.art_decode(qf, kf, vf, seq, inp.scale, tau, phi, patience, probe)
        nb = -(-int(seq[0]) // 64)
        oracle.decode_blocks(qf, kf, vf, seq, inp.scale, [[sorted(forced_blocks(nb, n_sink, win_recent))]])

    def timed(fn, items, budget):
        done, t0 = 0, time.perf_counter()
        for it in items:
            fn(it)
            done += 1
            if time.perf_counter() - t0 > budget:
                break
        return done, time.perf_counter() - t0

    done, el = timed(step_unit, range(B * Hkv), budget_s)
    with threadpool_limits(limits=1):
        done1, el1 = timed(step_unit, range(B * Hkv), budget_s / 3)
    res = {"value": round(done * bytes_per_unit / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"{done} of {B * Hkv} (batch row, KV head) units of the same input, every stage, "
                     f"float64 numpy, {el:.1f}s",
           "single_thread": {"value": round(done1 * bytes_per_unit / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                             "sample": f"{done1} units, every stage, {el1:.1f}s"}}

    # small fp32 single-head 4K workload: dense + top-8 (block 0 forced) selection + decode over it
    W1 = synth.WORKLOADS[1]
    t1 = synth.make_inputs(1, W1["B"], W1["Hq"], W1["Hkv"], W1["d"], W1["L"], dtype="f32", kind="gauss")
    q1, k1, v1 = t1.f64()

    def tiny(_):
        oracle.decode_dense(q1, k1, v1, t1.seq_lens, t1.scale)
        sig = oracle.centroid_scores(q1, oracle.block_centroids(k1, t1.seq_lens), t1.seq_lens, t1.scale)
        oracle.decode_blocks(q1, k1, v1, t1.seq_lens, t1.scale,
                             oracle.select_all(sig, t1.seq_lens, W1["topk"], W1["n_sink"], W1["n_recent"]))

    # 32K batch-8 dense: 8 units drawn on their own (the same values as the GPU's input), before timing
    W2 = synth.WORKLOADS[2]
    G2 = W2["Hq"] // W2["Hkv"]
    up = lambda a: synth.bf16_to_f32(a).astype(np.float64)
    units2 = [tuple(up(x) for x in synth.draw_unit(2, b, 0, G2, W2["d"], W2["L"], W2["L"], "bf16", W2["kind"]))
              for b in range(8)]

    def dense32k(u):
        qg, kk, vv = units2[u]
        oracle.decode_dense(qg[None], kk[None, None], vv[None, None], np.array([W2["L"]], dtype=np.int32),
                            1 / math.sqrt(W2["d"]))

    for name, fn, n, by in (("tiny4k", tiny, 20, W1["L"] * W1["d"] * 4 * 2),
                            ("dense32k_b8", dense32k, 8, W2["L"] * W2["d"] * 2 * 2)):
        row = {}
        for label, lim in (("threads", None), ("single_thread", 1)):
            if lim is None:
                k_, e_ = timed(fn, range(n), budget_s / 3)
            else:
                with threadpool_limits(limits=lim):
                    k_, e_ = timed(fn, range(n), budget_s / 3)
            row[label] = {"ms_per_item": round(1e3 * e_ / k_, 3), "gbs": round(k_ * by / e_ / 1e9, 4),
                          "items": k_}
        row["item"] = "one decode step" if name == "tiny4k" else "one (batch row, KV head) unit, dense"
        res[name] = row
    return res


if __name__ == "__main__":
    main()
