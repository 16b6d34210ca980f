"""GPU parity on the small fp32 configuration (one head, d 64, 4096 tokens,
top-8 blocks plus block 0), every stage of the path compared in full with
the oracle: dense split-KV decode and merge, centroid build, scores, top-k,
listed-block decode, a sink-only window, ART (default order, importance
order, over the selected list, across workgroups)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.art import art_margin_ok, importance_order
from oracle.selection import selection_gap
from tests.gpu_util import TOL, assert_close, assert_states_close, log, upload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS[1]


def tiny_inputs():
    B, Hq, Hkv, d, L = W["B"], W["Hq"], W["Hkv"], W["d"], W["L"]
    return synth.make_inputs(1, B, Hq, Hkv, d, L, dtype=W["dtype"], kind=W["kind"])


def test_tiny_fp32_dense_and_selection_path():
    import sparse_kv_amd as skv

    log("[tiny] fp32 d=64 4K: dense, centroids, scores, top-8 + block 0, listed-block decode")
    inp = tiny_inputs()
    q, k, v, sl = upload(inp)
    qf, kf, vf = inp.f64()
    ref = oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale)
    for S in (1, 4, 64):
        m, l, o = skv.attn_decode_dense(q, k, v, sl, num_splits=S)
        out = skv.attn_merge_states(m, l, o)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, TOL, f"dense S={S}")
        if S == 4:
            rm, rl, ro = oracle.decode_split_states(qf, kf, vf, inp.seq_lens, inp.scale, S)
            assert_states_close(m, l, o, rm, rl, ro, TOL, "dense split states")

    C = skv.attn_build_centroids(k, sl)
    sc = skv.attn_score_centroids(q, C, sl)
    topk, ns, nr = W["topk"], W["n_sink"], W["n_recent"]
    idx, n = skv.attn_select_topk(sc, sl, k=topk, n_sink_blocks=ns, n_recent_blocks=nr)
    torch.cuda.synchronize()
    RC = oracle.block_centroids(kf, inp.seq_lens)
    assert_close(C.cpu().numpy(), RC, 1e-5, "centroids")
    RS = oracle.centroid_scores(qf, RC, inp.seq_lens, inp.scale)
    assert_close(sc.cpu().numpy(), RS, 1e-5, "scores")
    nb = W["L"] // 64
    gap = selection_gap(RS[0, 0], nb, topk, ns, nr)
    assert gap > 1e-4, f"input lacks a selection margin ({gap})"
    sel = oracle.select_all(RS, inp.seq_lens, topk, ns, nr)
    assert len(sel[0][0]) == topk + 1 and sel[0][0][0] == 0
    assert int(n[0, 0]) == len(sel[0][0]) and idx[0, 0, :len(sel[0][0])].cpu().tolist() == sel[0][0]
    want = oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, sel)
    for S in (1, 2, 3, 9):
        m, l, o = skv.attn_decode_sparse(q, k, v, idx, n, sl, num_splits=S)
        out = skv.attn_merge_states(m, l, o)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), want, TOL, f"top-8 + block 0 decode S={S}")

    # sink-only window (k = 0, no recent blocks): attention over block 0 alone
    widx, wn = skv.attn_select_topk(None, sl, k=0, n_sink_blocks=1, n_recent_blocks=0, shape=(1, 1, nb), device="cuda")
    out = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, widx, wn, sl, num_splits=2))
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, [[[0]]]), TOL,
                 "block 0 only")


# (tau, phi, patience, expected stop): the configured thresholds never stop on
# these Gaussian inputs; looser ones stop part-way
ART_CASES = [(1e-3, 1e-4, 2, 63), (0.02, 0.02, 2, 20), (0.05, 0.05, 1, 9), (0.1, 0.1, 3, 8)]


@pytest.mark.parametrize("tau,phi,p,stop_at", ART_CASES)
def test_tiny_fp32_art(tau, phi, p, stop_at):
    import sparse_kv_amd as skv

    log(f"[tiny] fp32 d=64 4K ART tau={tau} phi={phi} p={p}")
    inp = tiny_inputs()
    q, k, v, sl = upload(inp)
    qf, kf, vf = inp.f64()
    probe = 8
    ro, rs, tr = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, tau, phi, p, probe)
    assert art_margin_ok(tr[(0, 0)], tau, phi), "input lacks ART decision margins"
    assert int(rs[0, 0]) == stop_at
    kw = dict(tau=tau, phi=phi, patience=p, probe_dim=probe)
    ws = torch.empty(max(skv.attn_art_workspace_bytes(q, k), 1), dtype=torch.uint8, device="cuda")
    for name, (out, stop, fetched) in (("one workgroup", skv.attn_decode_art(q, k, v, sl, **kw)),
                                       ("across workgroups", skv.attn_decode_art_ws(q, k, v, sl, workspace=ws, **kw))):
        torch.cuda.synchronize()
        assert int(stop[0, 0]) == stop_at, (name, int(stop[0, 0]))
        assert_close(out.cpu().numpy(), ro, TOL, f"ART {name}")
        assert stop_at + 1 <= int(fetched[0, 0]) <= 64, (name, int(fetched[0, 0]))

    # importance first: block 0, then blocks by descending centroid score
    sc = skv.attn_score_centroids(q, skv.attn_build_centroids(k, sl), sl)
    order = skv.attn_order_blocks(sc, sl)
    torch.cuda.synchronize()
    RS = oracle.centroid_scores(qf, oracle.block_centroids(kf, inp.seq_lens), inp.seq_lens, inp.scale)
    want_order = importance_order(RS[0, 0].astype(np.float32), 64)
    ranked = RS[0, 0][want_order[1:]]
    assert np.min(ranked[:-1] - ranked[1:]) > 1e-4, "input lacks an importance-order margin"
    assert order[0, 0].cpu().tolist() == want_order
    ro_i, rs_i, tr_i = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, tau, phi, p, probe,
                                         order=np.array(want_order)[None, None])
    assert art_margin_ok(tr_i[(0, 0)], tau, phi), "importance order lacks ART decision margins"
    out, stop, _ = skv.attn_decode_art(q, k, v, sl, order=order, **kw)
    torch.cuda.synchronize()
    assert int(stop[0, 0]) == int(rs_i[0, 0])
    assert_close(out.cpu().numpy(), ro_i, TOL, "importance-first ART")

    # ART over the top-8 + block 0 list, in list order
    idx, n = skv.attn_select_topk(sc, sl, k=W["topk"], n_sink_blocks=W["n_sink"], n_recent_blocks=W["n_recent"])
    torch.cuda.synchronize()
    lst = oracle.select_all(RS, inp.seq_lens, W["topk"], W["n_sink"], W["n_recent"])[0][0]
    assert idx[0, 0, :int(n[0, 0])].cpu().tolist() == lst
    ro_l, rs_l, tr_l = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, tau, phi, p, probe,
                                         order=np.array(lst + [0] * (64 - len(lst)))[None, None],
                                         n_visit=np.array([[len(lst)]]))
    assert art_margin_ok(tr_l[(0, 0)], tau, phi), "listed order lacks ART decision margins"
    for name, fn in (("one workgroup", skv.attn_decode_art_list), ("across workgroups", skv.attn_decode_art_list_ws)):
        extra = dict(workspace=ws) if fn is skv.attn_decode_art_list_ws else {}
        out, stop, _ = fn(q, k, v, idx, n, sl, **kw, **extra)
        torch.cuda.synchronize()
        assert int(stop[0, 0]) == int(rs_l[0, 0]), name
        assert_close(out.cpu().numpy(), ro_l, TOL, f"ART over the selected list, {name}")
