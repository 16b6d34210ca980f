"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark uses; the oracle checks sampled (batch row, KV head) units."""

import math
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.art import art_margin_ok
from oracle.selection import forced_blocks, selection_gap
from tests.gpu_util import TOL, assert_close, log

pytestmark = pytest.mark.gpu

SAMPLE = [(0, 0), (3, 5), (7, 7)]  # (batch row, KV head) units checked against the oracle


def up(a, dtype="bf16"):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def unit_f64(inp, b, g):
    G = inp.q.shape[1] // inp.k.shape[1]
    q = inp.upcast(inp.q[b:b + 1, g * G:(g + 1) * G])
    k = inp.upcast(inp.k[b:b + 1, g:g + 1])
    v = inp.upcast(inp.v[b:b + 1, g:g + 1])
    return q, k, v, inp.seq_lens[b:b + 1]


def test_llama_dense_32k_batch8_16_splits():
    W = synth.WORKLOADS[2]
    t = time.time()
    inp = synth.make_inputs(2, W["B"], W["Hq"], W["Hkv"], W["d"], W["L"], kind=W["kind"])
    log(f"[full] dense 32K batch 8: inputs in {time.time() - t:.1f}s")
    import sparse_kv_amd as skv

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    out = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, None, num_splits=W["splits"]))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = W["Hq"] // W["Hkv"]
    for b, g in SAMPLE:
        qf, kf, vf, seq = unit_f64(inp, b, g)
        ref = oracle.decode_dense(qf, kf, vf, seq, inp.scale)
        assert_close(out[b, g * G:(g + 1) * G], ref[0], TOL, f"unit ({b},{g})")


def test_sparse_128k_batch8_selection_and_dense():
    W = synth.WORKLOADS[3]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    k_top, ns, nr = W["topk"], W["n_sink"], W["n_recent"]
    t = time.time()
    inp = synth.make_inputs(3, B, Hq, Hkv, d, L, kind="mixture")
    log(f"[full] 128K batch 8: inputs in {time.time() - t:.1f}s")
    import sparse_kv_amd as skv

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    dense = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, None, num_splits=4))  # the benchmark's launch
    C = skv.attn_build_centroids(k)
    sc = skv.attn_score_centroids(q, C)
    idx, n = skv.attn_select_topk(sc, None, k=k_top, n_sink_blocks=ns, n_recent_blocks=nr)
    sp = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, None, num_splits=4))  # the benchmark's launch
    # the sink + window stage: block 0 and the last 128 blocks, 4 splits
    widx, wn = skv.attn_select_topk(None, None, k=0, n_sink_blocks=1, n_recent_blocks=128, shape=(B, Hkv, L // 64),
                                    device="cuda")
    win = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, widx, wn, None, num_splits=4))
    torch.cuda.synchronize()
    dense, sp, idx, n = dense.cpu().numpy(), sp.cpu().numpy(), idx.cpu().numpy(), n.cpu().numpy()
    win = win.cpu().numpy()
    window = [0] + list(range(L // 64 - 128, L // 64))
    assert (wn.cpu().numpy() == 129).all() and (widx.cpu().numpy()[:, :, :129] == np.array(window)).all()
    assert (n == ns + nr + k_top).all()
    G = Hq // Hkv
    checked = 0
    for b, g in SAMPLE:
        qf, kf, vf, seq = unit_f64(inp, b, g)
        assert_close(dense[b, g * G:(g + 1) * G], oracle.decode_dense(qf, kf, vf, seq, inp.scale)[0], TOL,
                     f"dense unit ({b},{g})")
        sig = oracle.centroid_scores(qf, oracle.block_centroids(kf, seq), seq, inp.scale)
        gap = selection_gap(sig[0, 0], L // 64, k_top, ns, nr)
        lists = oracle.select_all(sig, seq, k_top, ns, nr)
        log(f"  unit ({b},{g}): top-k boundary gap {gap:.2e}")
        if gap > 1e-4:
            assert idx[b, g, :n[b, g]].tolist() == lists[0][0], f"selected blocks of unit ({b},{g})"
            checked += 1
        got = [[idx[b, g, :n[b, g]].tolist()]]
        ref = oracle.decode_blocks(qf, kf, vf, seq, inp.scale, got)
        assert_close(sp[b, g * G:(g + 1) * G], ref[0], TOL, f"sparse unit ({b},{g})")
        assert_close(win[b, g * G:(g + 1) * G], oracle.decode_blocks(qf, kf, vf, seq, inp.scale, [[window]])[0], TOL,
                     f"sink + window unit ({b},{g})")
    assert checked >= 2, "too few sampled units with a clear top-k margin"


def test_art_64k_batch32_stop_positions():
    W = synth.WORKLOADS[4]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    t = time.time()
    inp = synth.make_inputs(4, B, Hq, Hkv, d, L, kind="recency")
    log(f"[full] ART 64K batch 32: inputs in {time.time() - t:.1f}s")
    import sparse_kv_amd as skv

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    out, stop, fetched = skv.attn_decode_art(q, k, v, None, tau=W["tau"], phi=W["phi"], patience=W["patience"],
                                             probe_dim=W["probe_dim"])
    torch.cuda.synchronize()
    out, stop, fetched = out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()
    G = Hq // Hkv
    log(f"  mean stop {stop.mean():.2f}, mean blocks fetched {fetched.mean():.2f}")
    for b, g in SAMPLE + [(31, 0), (16, 3)]:
        qf, kf, vf, seq = unit_f64(inp, b, g)
        ro, rs, tr = oracle.art_decode(qf, kf, vf, seq, inp.scale, W["tau"], W["phi"], W["patience"], W["probe_dim"])
        assert all(art_margin_ok(x, W["tau"], W["phi"]) for x in tr.values()), f"unit ({b},{g}) lacks margins"
        assert stop[b, g * G:(g + 1) * G].tolist() == rs[0].tolist(), f"stop positions of unit ({b},{g})"
        assert_close(out[b, g * G:(g + 1) * G], ro[0], TOL, f"ART unit ({b},{g})")
        need = int(rs.max()) + 1
        assert need <= fetched[b, g] <= need + 8, (b, g, need, fetched[b, g])


def test_art_128k_batch8_across_workgroups():
    """ART in the benchmark's 128K batch-8 configuration (block 0, then newest
    first), through attn_decode_art_ws: 64 (b, kv head) units, each streamed
    by several workgroups.  Units whose every decision clears the margins are
    checked exactly against the oracle; all units against the one-workgroup
    kernel (same stops wherever both clear the margins, outputs to TOL)."""
    W3, W4 = synth.WORKLOADS[3], synth.WORKLOADS[4]
    B, Hq, Hkv, d, L = W3["B"], W3["Hq"], W3["Hkv"], W3["d"], W3["L"]
    tau, phi, p, probe = W4["tau"], W4["phi"], W4["patience"], W4["probe_dim"]
    t = time.time()
    inp = synth.make_inputs(3, B, Hq, Hkv, d, L, kind="mixture")
    log(f"[full] ART 128K batch 8 across workgroups: inputs in {time.time() - t:.1f}s")
    import sparse_kv_amd as skv

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    kw = dict(tau=tau, phi=phi, patience=p, probe_dim=probe)
    ws = torch.empty(skv.attn_art_workspace_bytes(q, k), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    out, stop, fetched = skv.attn_decode_art_ws(q, k, v, None, workspace=ws, **kw)
    out1, stop1, fetched1 = skv.attn_decode_art(q, k, v, None, **kw)
    torch.cuda.synchronize()
    out, stop, fetched = out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()
    out1, stop1 = out1.cpu().numpy(), stop1.cpu().numpy()
    G = Hq // Hkv
    log(f"  mean stop {stop.mean():.1f}, max {stop.max()}, mean fetched {fetched.mean():.1f} "
        f"(one workgroup: {fetched1.float().mean().item():.1f}); {int((stop == stop1).sum())} of {stop.size} "
        f"stops equal the one-workgroup kernel's")
    units = SAMPLE + [(b, g) for b in range(B) for g in range(Hkv) if (b, g) not in SAMPLE]
    checked = 0
    for b, g in units:
        qf, kf, vf, seq = unit_f64(inp, b, g)
        ro, rs, tr = oracle.art_decode(qf, kf, vf, seq, inp.scale, tau, phi, p, probe)
        if not all(art_margin_ok(x, tau, phi) for x in tr.values()):
            continue
        assert stop[b, g * G:(g + 1) * G].tolist() == rs[0].tolist(), f"stop positions of unit ({b},{g})"
        assert stop1[b, g * G:(g + 1) * G].tolist() == rs[0].tolist(), f"one-workgroup stops of unit ({b},{g})"
        assert_close(out[b, g * G:(g + 1) * G], ro[0], TOL, f"ART unit ({b},{g})")
        need = int(rs.max()) + 1
        assert need <= fetched[b, g] <= need + min(128, max(64, need)), (b, g, need, fetched[b, g])
        checked += 1
        if checked == 3:
            break
    assert checked >= 2, "too few units clear the ART decision margins"
    same = stop == stop1
    for b in range(B):
        for g in range(Hkv):
            if same[b, g * G:(g + 1) * G].all():
                assert_close(out[b, g * G:(g + 1) * G], out1[b, g * G:(g + 1) * G], TOL, f"unit ({b},{g}) vs one")
    assert same.mean() > 0.9


def test_routed_36_layer_stack_256k():
    W = synth.WORKLOADS[5]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    nb = L // 64
    mask = synth.route_mask(W["n_layers"], W["n_full"])
    import sparse_kv_amd as skv

    keep = [[sorted(forced_blocks(nb, W["n_sink"], W["n_recent"]))] * Hkv]
    t = time.time()
    qs, ks, vs, host = [], [], [], {}
    check = {int(np.flatnonzero(mask == 1)[0]), int(np.flatnonzero(mask == 0)[0])}
    for i in range(W["n_layers"]):
        inp = synth.make_inputs(5, B, Hq, Hkv, d, L, kind="needles", layer=i)
        if i in check:
            host[i] = (unit_f64(inp, 0, 2), unit_f64(inp, 0, 6))  # clean copies, before any poisoning
        if not mask[i]:
            synth.poison_blocks(inp, keep)  # a sink + window layer must never read these
        qs.append(up(inp.q))
        ks.append(up(inp.k))
        vs.append(up(inp.v))
        del inp
    log(f"[full] 36-layer 256K stack: inputs in {time.time() - t:.1f}s")
    sa_idx, sa_n = skv.attn_select_topk(None, None, k=0, n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"],
                                        shape=(B, Hkv, nb), device="cuda")
    # the benchmark's launch configuration: 8 shards x 4 splits, 32 splits for sink + window layers
    outs = skv.attn_decode_routed(qs, ks, vs, mask, None, n_shards=W["n_shards"], splits_per_shard=4,
                                  sa_block_idx=sa_idx, sa_n_sel=sa_n, sa_splits=32)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for i in sorted(check):
        for (qf, kf, vf, seq), g in zip(host[i], (2, 6)):
            if mask[i]:
                ref = oracle.decode_dense(qf, kf, vf, seq, 1 / math.sqrt(d))
            else:
                ref = oracle.decode_blocks(qf, kf, vf, seq, 1 / math.sqrt(d), [[keep[0][0]]])
            assert_close(outs[i][0, g * G:(g + 1) * G].cpu().numpy(), ref[0], TOL,
                         f"layer {i} ({'FA' if mask[i] else 'SA'}) kv head {g}")
    for o in outs:
        assert torch.isfinite(o).all()


def test_importance_first_art_128k_batch8():
    """Centroid scores -> importance order -> ART at 128K batch 8 (mixture keys).

    The order kernel's result is checked as a descending sort of the oracle's
    float64 scores; stop positions and outputs are checked exactly with the
    oracle's own order placed in the sampled rows."""
    W3, W4 = synth.WORKLOADS[3], synth.WORKLOADS[4]
    B, Hq, Hkv, d, L = W3["B"], W3["Hq"], W3["Hkv"], W3["d"], W3["L"]
    tau, phi, p, probe = W4["tau"], W4["phi"], W4["patience"], W4["probe_dim"]
    nb = L // 64
    t = time.time()
    inp = synth.make_inputs(3, B, Hq, Hkv, d, L, kind="mixture")
    log(f"[full] importance-first ART 128K batch 8: inputs in {time.time() - t:.1f}s")
    import sparse_kv_amd as skv

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    order = skv.attn_order_blocks(skv.attn_score_centroids(q, skv.attn_build_centroids(k)))
    out, stop, fetched = skv.attn_decode_art(q, k, v, None, order=order, tau=tau, phi=phi, patience=p,
                                             probe_dim=probe)
    torch.cuda.synchronize()
    order_h = order.cpu().numpy()
    log(f"  GPU chain: mean stop {stop.float().mean().item():.1f}, mean blocks fetched "
        f"{fetched.float().mean().item():.1f} of {nb}")
    G = Hq // Hkv
    # every ART decision of a checked unit must clear a 1% band around the
    # thresholds; scan units in a fixed order until three do
    units = SAMPLE + [(b, g) for b in range(B) for g in range(Hkv) if (b, g) not in SAMPLE]
    oracle_rows, ref = {}, {}
    for i, (b, g) in enumerate(units):
        qf, kf, vf, seq = unit_f64(inp, b, g)
        sc = oracle.centroid_scores(qf, oracle.block_centroids(kf, seq), seq, inp.scale)[0, 0]
        o = order_h[b, g]
        assert o[0] == 0 and sorted(o.tolist()) == list(range(nb)), f"unit ({b},{g}) order is no permutation"
        assert np.min(sc[o[1:-1]] - sc[o[2:]]) > -1e-4, f"unit ({b},{g}) order is not descending"
        oo = oracle.importance_order(sc.astype(np.float32), nb)
        ro, rs, tr = oracle.art_decode(qf, kf, vf, seq, inp.scale, tau, phi, p, probe, order=[[oo]])
        if all(art_margin_ok(x, tau, phi) for x in tr.values()):
            oracle_rows[(b, g)] = oo
            ref[(b, g)] = (ro[0], rs[0])
            if len(ref) == 3:
                break
    log(f"  {len(ref)} of {i + 1} scanned units clear the ART decision margins")
    assert len(ref) >= 2
    inj = order_h.copy()
    for (b, g), oo in oracle_rows.items():
        inj[b, g] = oo
    inj_d = torch.from_numpy(inj).cuda()
    kw = dict(order=inj_d, tau=tau, phi=phi, patience=p, probe_dim=probe)
    # one workgroup per unit, and the benchmark's path: several workgroups per unit
    for name, fn in (("one", skv.attn_decode_art), ("ws", skv.attn_decode_art_ws)):
        out2, stop2, _ = fn(q, k, v, None, **kw)
        torch.cuda.synchronize()
        out2, stop2 = out2.cpu().numpy(), stop2.cpu().numpy()
        for (b, g), (ro, rs) in ref.items():
            assert stop2[b, g * G:(g + 1) * G].tolist() == rs.tolist(), f"{name}: stop positions of unit ({b},{g})"
            assert_close(out2[b, g * G:(g + 1) * G], ro, TOL, f"{name}: importance-first ART unit ({b},{g})")


def test_two_level_selection_128k_batch8():
    """Two-level selection at 128K batch 8 (super-blocks of 16 blocks, 32 opened,
    205 picks + sink + 64-block window) and decode over its lists."""
    from oracle.selection import select_blocks_two_level, super_centroids, two_level_gaps

    W = synth.WORKLOADS[3]
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    k_top, ns, nr = W["topk"], W["n_sink"], W["n_recent"]
    group, kc = 16, 32
    inp = synth.make_inputs(3, B, Hq, Hkv, d, L, kind="mixture")
    import sparse_kv_amd as skv

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    C = skv.attn_build_centroids(k)
    C2 = skv.attn_build_super_centroids(C, group)
    idx, n = skv.attn_select_two_level(q, C, C2, group, None, k_coarse=kc, k=k_top, n_sink_blocks=ns, n_recent_blocks=nr)
    sp = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, None, num_splits=4))
    torch.cuda.synchronize()
    idx, n, sp = idx.cpu().numpy(), n.cpu().numpy(), sp.cpu().numpy()
    assert (n == ns + nr + k_top).all()
    G = Hq // Hkv
    nb = L // 64
    checked = 0
    for b, g in SAMPLE:
        qf, kf, vf, seq = unit_f64(inp, b, g)
        fine = oracle.centroid_scores(qf, oracle.block_centroids(kf, seq), seq, inp.scale)[0, 0]
        coarse = oracle.centroid_scores(qf, super_centroids(kf, seq, group), seq, inp.scale, block=64 * group)[0, 0]
        cg, fg = two_level_gaps(fine, coarse, nb, group, kc, k_top, ns, nr)
        log(f"  unit ({b},{g}): coarse gap {cg:.2e}, fine gap {fg:.2e}")
        if min(cg, fg) > 1e-4:
            ref = select_blocks_two_level(fine, coarse, nb, group, kc, k_top, ns, nr)
            assert idx[b, g, :n[b, g]].tolist() == ref, f"two-level blocks of unit ({b},{g})"
            checked += 1
        got = [[idx[b, g, :n[b, g]].tolist()]]
        assert_close(sp[b, g * G:(g + 1) * G], oracle.decode_blocks(qf, kf, vf, seq, inp.scale, got)[0], TOL,
                     f"decode over the two-level list, unit ({b},{g})")
    assert checked >= 2, "too few sampled units with clear two-level margins"
