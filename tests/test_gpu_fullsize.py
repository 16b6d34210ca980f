"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark uses.  Every (batch row, KV head) unit is compared with the oracle.

The inputs are the benchmark's: units whose decisions would fall inside the
margins are drawn from later sub-seeds (tests/golden/redraws.json, written by
tests/golden/make_redraws.py from the oracle alone), so every selected-block
list and every ART stop position is compared exactly, and every output to
the max-abs tolerance."""

import math
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.art import art_margin_ok, default_order, importance_order
from oracle.selection import (forced_blocks, select_blocks, select_blocks_two_level, selection_gap, super_centroids,
                              two_level_gaps)
from tests.gpu_util import TOL, assert_close, log

pytestmark = pytest.mark.gpu

THREADS = 8  # oracle units in flight (numpy releases the GIL in its array work)


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def f64(a):
    return synth.bf16_to_f32(a).astype(np.float64)


def unit_f64(inp, b, g):
    """float64 (q [1, G, d], k [1, 1, L, d], v [1, 1, L, d], seq [1]) of one unit."""
    G = inp.q.shape[1] // inp.k.shape[1]
    return (f64(inp.q[b:b + 1, g * G:(g + 1) * G]), f64(inp.k[b:b + 1, g:g + 1]), f64(inp.v[b:b + 1, g:g + 1]),
            inp.seq_lens[b:b + 1])


def per_unit(fn, units):
    with ThreadPoolExecutor(THREADS) as ex:
        return dict(zip(units, ex.map(fn, units)))


_cache = {}


def workload(cfg):
    """(host inputs, device q, k, v) of a full-size workload; one workload is kept at a time."""
    if cfg not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        t = time.time()
        inp = synth.workload_inputs(cfg)
        dev = (up(inp.q), up(inp.k), up(inp.v))
        log(f"[full] {synth.WORKLOADS[cfg]['name']}: inputs in {time.time() - t:.1f}s, "
            f"{len(synth.redraws(synth.WORKLOADS[cfg].get('redraws', '')))} units redrawn")
        _cache[cfg] = (inp, dev)
    return _cache[cfg]


# ---------------------------------------------------------------- 32K batch 8
@pytest.mark.parametrize("splits", [16, 4])
def test_dense_32k_batch8_every_unit(splits):
    """Dense split-KV decode + merge at 32K, batch 8 (needle keys): 16 splits as the
    workload states, 4 as the benchmark launches it."""
    import sparse_kv_amd as skv

    W = synth.WORKLOADS[2]
    inp, (q, k, v) = workload(2)
    out = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, None, num_splits=splits)).cpu().numpy()
    G = W["Hq"] // W["Hkv"]
    units = [(b, g) for b in range(W["B"]) for g in range(W["Hkv"])]

    def ref(u):
        qf, kf, vf, seq = unit_f64(inp, *u)
        return oracle.decode_dense(qf, kf, vf, seq, inp.scale)[0]

    refs = per_unit(ref, units)
    err = max(float(np.abs(out[b, g * G:(g + 1) * G] - refs[(b, g)]).max()) for b, g in units)
    log(f"  {len(units)} units, {splits} splits: max-abs error {err:.3e}")
    assert np.isfinite(out).all() and err <= TOL


# --------------------------------------------------------------- 128K batch 8
_ref128 = {}


def oracle_128k():
    """Every oracle result the 128K batch-8 tests compare with, per unit, computed once."""
    if _ref128:
        return _ref128
    W = synth.WORKLOADS[3]
    inp, _ = workload(3)
    nb = W["L"] // 64
    art = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])
    ks, ns, nr, grp, kc = W["topk"], W["n_sink"], W["n_recent"], W["group"], W["k_coarse"]

    def one(u):
        qf, kf, vf, seq = unit_f64(inp, *u)
        r = {"dense": oracle.decode_dense(qf, kf, vf, seq, inp.scale)[0]}
        sig = oracle.centroid_scores(qf, oracle.block_centroids(kf, seq), seq, inp.scale)[0, 0]
        coarse = oracle.centroid_scores(qf, super_centroids(kf, seq, grp), seq, inp.scale, block=64 * grp)[0, 0]
        r["gap"] = selection_gap(sig, nb, ks, ns, nr)
        r["gaps2"] = two_level_gaps(sig, coarse, nb, grp, kc, ks, ns, nr)
        r["list"] = select_blocks(sig, nb, ks, ns, nr)
        r["sparse"] = oracle.decode_blocks(qf, kf, vf, seq, inp.scale, [[r["list"]]])[0]
        r["window"] = oracle.decode_blocks(qf, kf, vf, seq, inp.scale,
                                           [[sorted(forced_blocks(nb, ns, W["win_recent"]))]])[0]
        r["list2"] = select_blocks_two_level(sig, coarse, nb, grp, kc, ks, ns, nr)
        r["sparse2"] = oracle.decode_blocks(qf, kf, vf, seq, inp.scale, [[r["list2"]]])[0]
        r["scores"] = sig
        r["order"] = importance_order(sig.astype(np.float32), nb)
        for name, order, n_visit in (("art", None, None), ("art_imp", [[r["order"]]], None),
                                     ("art_sel", [[r["list"] + [0] * (nb - len(r["list"]))]], [[len(r["list"])]])):
            o, s, tr = oracle.art_decode(qf, kf, vf, seq, inp.scale, order=order, n_visit=n_visit, **art)
            r[name] = (o[0], s[0], all(art_margin_ok(x, W["tau"], W["phi"]) for x in tr.values()))
        return r

    t = time.time()
    units = [(b, g) for b in range(W["B"]) for g in range(W["Hkv"])]
    _ref128.update(per_unit(one, units))
    log(f"  oracle over all {len(units)} units of the 128K batch-8 input in {time.time() - t:.1f}s")
    return _ref128


def check_units(got, key, what, units=None):
    """got [B, Hq, d] against the oracle's per-unit `key` output on every unit."""
    refs = oracle_128k()
    G = got.shape[1] // 8
    worst = 0.0
    for (b, g) in (units or refs):
        ref = refs[(b, g)][key]
        ref = ref[0] if isinstance(ref, tuple) else ref
        worst = max(worst, float(np.abs(got[b, g * G:(g + 1) * G] - ref).max()))
    log(f"  {what}: {len(units or refs)} units, max-abs error {worst:.3e}")
    assert np.isfinite(got).all() and worst <= TOL, what


def test_128k_batch8_margins_hold():
    """The redrawn input leaves every decision of every unit clear of its margin."""
    refs = oracle_128k()
    bad = [u for u, r in refs.items()
           if not (r["gap"] > 1e-4 and min(r["gaps2"]) > 1e-4 and r["art"][2] and r["art_imp"][2] and r["art_sel"][2])]
    assert not bad, f"units without decision margins: {bad}"


def test_128k_batch8_dense_selection_sparse_window():
    """Dense (4 splits), centroids -> scores -> top-k (205 + sink + 64 recent) -> listed-block
    decode (3 splits), and the sink + 128-block window (3 splits): every unit."""
    import sparse_kv_amd as skv

    W = synth.WORKLOADS[3]
    B, Hkv, nb = W["B"], W["Hkv"], W["L"] // 64
    inp, (q, k, v) = workload(3)
    dense = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, None, num_splits=4))
    C = skv.attn_build_centroids(k)
    sc = skv.attn_score_centroids(q, C)
    idx, n = skv.attn_select_topk(sc, None, k=W["topk"], n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"])
    sp = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, None, num_splits=3))
    widx, wn = skv.attn_select_topk(None, None, k=0, n_sink_blocks=W["n_sink"], n_recent_blocks=W["win_recent"],
                                    shape=(B, Hkv, nb), device="cuda")
    win = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, widx, wn, None, num_splits=3))
    torch.cuda.synchronize()
    refs = oracle_128k()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    for (b, g), r in refs.items():
        assert idx[b, g, :n[b, g]].tolist() == r["list"], f"selected blocks of unit ({b},{g})"
        assert (idx[b, g, n[b, g]:] == -1).all()
    window = sorted(forced_blocks(nb, W["n_sink"], W["win_recent"]))
    assert (wn.cpu().numpy() == len(window)).all() and (widx.cpu().numpy() == np.array(window)).all()
    scg = sc.cpu().numpy()
    worst = max(float(np.abs(scg[b, g] - r["scores"]).max()) for (b, g), r in refs.items())
    log(f"  centroid scores: max-abs error {worst:.3e}")
    assert worst < 1e-4
    check_units(dense.cpu().numpy(), "dense", "dense")
    check_units(sp.cpu().numpy(), "sparse", "top-k listed-block decode")
    check_units(win.cpu().numpy(), "window", "sink + window decode")


def test_128k_batch8_two_level_selection():
    """Super-blocks of 16 blocks, 32 opened, 205 picks + sink + 64 recent; decode over the lists."""
    import sparse_kv_amd as skv

    W = synth.WORKLOADS[3]
    inp, (q, k, v) = workload(3)
    C = skv.attn_build_centroids(k)
    C2 = skv.attn_build_super_centroids(C, W["group"])
    idx, n = skv.attn_select_two_level(q, C, C2, W["group"], None, k_coarse=W["k_coarse"], k=W["topk"],
                                       n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"])
    sp = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, None, num_splits=3))
    torch.cuda.synchronize()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    for (b, g), r in oracle_128k().items():
        assert idx[b, g, :n[b, g]].tolist() == r["list2"], f"two-level blocks of unit ({b},{g})"
    check_units(sp.cpu().numpy(), "sparse2", "decode over the two-level lists")


def art_paths():
    import sparse_kv_amd as skv

    return (("one workgroup", skv.attn_decode_art), ("across workgroups", skv.attn_decode_art_ws))


def check_stops(stop, fetched, key, what, nv):
    """Exact stop positions on every unit; blocks fetched within the read-ahead bound."""
    refs = oracle_128k()
    G = stop.shape[1] // 8
    for (b, g), r in refs.items():
        assert stop[b, g * G:(g + 1) * G].tolist() == r[key][1].tolist(), f"{what}: stops of unit ({b},{g})"
        need = int(r[key][1].max()) + 1
        assert need <= fetched[b, g] <= min(nv, need + 128), f"{what}: unit ({b},{g}) fetched {fetched[b, g]}"
    log(f"  {what}: stops of all {len(refs)} units exact (mean {stop.mean():.1f}, max {stop.max()}); "
        f"fetched {fetched.mean():.1f} per unit")


def test_128k_batch8_art_recency_first():
    """ART (block 0, then newest first; tau 1e-3, phi 1e-4, p 2, probe 8), both launch forms."""
    W = synth.WORKLOADS[3]
    inp, (q, k, v) = workload(3)
    kw = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])
    for name, fn in art_paths():
        out, stop, fetched = fn(q, k, v, None, **kw)
        torch.cuda.synchronize()
        check_stops(stop.cpu().numpy(), fetched.cpu().numpy(), "art", f"recency-first ART, {name}", W["L"] // 64)
        check_units(out.cpu().numpy(), "art", f"recency-first ART output, {name}")


def test_128k_batch8_art_importance_first():
    """Centroid scores -> importance order -> ART.  The order kernel's rows equal the
    oracle's (block 0, then descending float32 score); ART runs on the GPU's own order
    (the benchmark's chain) and on the oracle's order written into the rows."""
    import sparse_kv_amd as skv

    W = synth.WORKLOADS[3]
    B, Hkv, nb = W["B"], W["Hkv"], W["L"] // 64
    inp, (q, k, v) = workload(3)
    refs = oracle_128k()
    order = skv.attn_order_blocks(skv.attn_score_centroids(q, skv.attn_build_centroids(k)))
    torch.cuda.synchronize()
    order_h = order.cpu().numpy()
    # blocks whose float32 scores differ by about a rounding step may trade places;
    # ART's result depends only on the positions it folds, 0 .. T
    same = {}
    for (b, g), r in refs.items():
        o = order_h[b, g]
        assert o[0] == 0 and sorted(o.tolist()) == list(range(nb)), f"unit ({b},{g}): order is no permutation"
        sc = r["scores"][o[1:]]
        assert np.min(sc[:-1] - sc[1:]) > -1e-4, f"unit ({b},{g}): order is not descending"
        T = int(r["art_imp"][1].max())
        same[(b, g)] = o[:T + 1].tolist() == r["order"][:T + 1]
    log(f"  order rows equal to the oracle's over the folded positions: {sum(same.values())} of {len(same)}")
    assert sum(same.values()) >= len(same) // 2
    ref_order = torch.from_numpy(np.array([[refs[(b, g)]["order"] for g in range(Hkv)] for b in range(B)],
                                          dtype=np.int32)).cuda()
    kw = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])
    for name, fn in art_paths():
        out, stop, fetched = fn(q, k, v, None, order=ref_order, **kw)
        torch.cuda.synchronize()
        check_stops(stop.cpu().numpy(), fetched.cpu().numpy(), "art_imp", f"importance-first ART, {name}", nb)
        check_units(out.cpu().numpy(), "art_imp", f"importance-first ART output, {name}")
        out, stop, _ = fn(q, k, v, None, order=order, **kw)
        torch.cuda.synchronize()
        stop = stop.cpu().numpy()
        units = [u for u, s in same.items() if s]
        for (b, g) in units:
            assert stop[b, g * 4:(g + 1) * 4].tolist() == refs[(b, g)]["art_imp"][1].tolist(), (name, b, g)
        check_units(out.cpu().numpy(), "art_imp", f"GPU chain scores -> order -> ART, {name}", units)


def test_128k_batch8_art_over_topk_lists():
    """ART over each unit's top-k list (205 + sink + 64 recent, ascending, so block 0
    first) -- the benchmark's art_sel stage -- on a copy of the cache whose unlisted
    blocks hold NaN, through both list entry points."""
    import sparse_kv_amd as skv

    W = synth.WORKLOADS[3]
    B, Hkv, L, d = W["B"], W["Hkv"], W["L"], W["d"]
    nb = L // 64
    inp, (q, k, v) = workload(3)
    refs = oracle_128k()
    sc = skv.attn_score_centroids(q, skv.attn_build_centroids(k))
    idx, n = skv.attn_select_topk(sc, None, k=W["topk"], n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"])
    torch.cuda.synchronize()
    idx_h, n_h = idx.cpu().numpy(), n.cpu().numpy()
    listed = np.zeros((B, Hkv, nb), dtype=bool)
    for (b, g), r in refs.items():
        assert idx_h[b, g, :n_h[b, g]].tolist() == r["list"]
        listed[b, g, r["list"]] = True
    unl = torch.from_numpy(~listed).cuda()
    kp, vp = k.clone(), v.clone()
    kp.view(B, Hkv, nb, 64, d)[unl] = float("nan")
    vp.view(B, Hkv, nb, 64, d)[unl] = float("nan")
    kw = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])
    n_list = int(n_h.max())
    for name, fn in (("one workgroup", skv.attn_decode_art_list), ("across workgroups", skv.attn_decode_art_list_ws)):
        out, stop, fetched = fn(q, kp, vp, idx, n, None, **kw)
        torch.cuda.synchronize()
        stop_h = stop.cpu().numpy()
        check_stops(stop_h, fetched.cpu().numpy(), "art_sel", f"ART over top-k lists, {name}", n_list)
        assert (stop_h < n_list - 1).mean() > 0.5, "most heads should stop inside their list"
        check_units(out.cpu().numpy(), "art_sel", f"ART over top-k lists output, {name}")
    del kp, vp


# --------------------------------------------------------------- 64K batch 32
def test_art_64k_batch32_every_unit():
    """ART at 64K, batch 32 (recency-concentrated keys): 256 units, one workgroup each
    (the benchmark's launch); every stop exact, every output within tolerance."""
    import sparse_kv_amd as skv

    W = synth.WORKLOADS[4]
    B, Hq, Hkv, L = W["B"], W["Hq"], W["Hkv"], W["L"]
    G = Hq // Hkv
    inp, (q, k, v) = workload(4)
    kw = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])
    out, stop, fetched = skv.attn_decode_art(q, k, v, None, **kw)
    torch.cuda.synchronize()
    out, stop, fetched = out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()
    units = [(b, g) for b in range(B) for g in range(Hkv)]

    def ref(u):
        qf, kf, vf, seq = unit_f64(inp, *u)
        o, s, tr = oracle.art_decode(qf, kf, vf, seq, inp.scale, **kw)
        return o[0], s[0], all(art_margin_ok(x, W["tau"], W["phi"]) for x in tr.values())

    t = time.time()
    refs = per_unit(ref, units)
    log(f"  oracle over {len(units)} units in {time.time() - t:.1f}s; mean stop {stop.mean():.2f}, "
        f"mean fetched {fetched.mean():.2f}")
    worst = 0.0
    for (b, g), (ro, rs, ok) in refs.items():
        assert ok, f"unit ({b},{g}) lacks ART decision margins"
        assert stop[b, g * G:(g + 1) * G].tolist() == rs.tolist(), f"stops of unit ({b},{g})"
        worst = max(worst, float(np.abs(out[b, g * G:(g + 1) * G] - ro).max()))
        need = int(rs.max()) + 1
        assert need <= fetched[b, g] <= need + 8, (b, g, need, fetched[b, g])
    log(f"  outputs: max-abs error {worst:.3e}")
    assert np.isfinite(out).all() and worst <= TOL


# ------------------------------------------------------ 36-layer stack at 256K
def test_routed_36_layer_stack_256k():
    """The 36-layer routed stack at 256K, batch 1, in the benchmark's launch configuration
    (8 shards x 4 splits; 32 splits for sink + window layers, whose other blocks hold NaN).
    Every KV head of two full-attention and two sink + window layers is checked; every
    layer's output is finite."""
    import sparse_kv_amd as skv

    _cache.clear()
    W = synth.WORKLOADS[5]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    G, nb = Hq // Hkv, L // 64
    mask = synth.route_mask(W["n_layers"], W["n_full"])
    keep = sorted(forced_blocks(nb, W["n_sink"], W["n_recent"]))
    check = [int(i) for i in np.flatnonzero(mask == 1)[:2]] + [int(i) for i in np.flatnonzero(mask == 0)[:2]]
    t = time.time()
    qs, ks, vs, host = [], [], [], {}
    for i in range(W["n_layers"]):
        inp = synth.make_inputs(5, B, Hq, Hkv, d, L, kind="needles", layer=i)
        if i in check:
            host[i] = synth.DecodeInputs(inp.q.copy(), inp.k.copy(), inp.v.copy(), inp.seq_lens, inp.dtype)
        if not mask[i]:
            synth.poison_blocks(inp, [[keep] * Hkv])  # a sink + window layer must never read these
        qs.append(up(inp.q))
        ks.append(up(inp.k))
        vs.append(up(inp.v))
        del inp
    log(f"[full] 36-layer 256K stack: inputs in {time.time() - t:.1f}s; checking layers {check}")
    sa_idx, sa_n = skv.attn_select_topk(None, None, k=0, n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"],
                                        shape=(B, Hkv, nb), device="cuda")
    outs = skv.attn_decode_routed(qs, ks, vs, mask, None, n_shards=W["n_shards"], splits_per_shard=4,
                                  sa_block_idx=sa_idx, sa_n_sel=sa_n, sa_splits=32)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.isfinite(o).all()

    def ref(job):
        i, g = job
        qf, kf, vf, seq = unit_f64(host[i], 0, g)
        if mask[i]:
            return oracle.decode_dense(qf, kf, vf, seq, 1 / math.sqrt(d))[0]
        return oracle.decode_blocks(qf, kf, vf, seq, 1 / math.sqrt(d), [[keep]])[0]

    refs = per_unit(ref, [(i, g) for i in check for g in range(Hkv)])
    for (i, g), r in refs.items():
        got = outs[i][0, g * G:(g + 1) * G].cpu().numpy()
        assert float(np.abs(got - r).max()) <= TOL, f"layer {i} ({'FA' if mask[i] else 'SA'}) kv head {g}"
    worst = max(float(np.abs(outs[i][0, g * G:(g + 1) * G].cpu().numpy() - r).max()) for (i, g), r in refs.items())
    log(f"  {len(refs)} (layer, KV head) pairs: max-abs error {worst:.3e}")
    del qs, ks, vs, outs
    torch.cuda.empty_cache()
