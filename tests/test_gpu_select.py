"""GPU parity: centroids, scores, top-k selection and listed-block decode."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.selection import selection_gap
from tests.gpu_util import TOL, assert_close, assert_states_close, log, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,d,seq", [("bf16", 128, [64 * 21, 64 * 7 + 9]), ("f32", 64, [64 * 21, 1]),
                                     ("bf16", 64, [0, 64 * 21]), ("f32", 128, [64 * 21, 64 * 3])])
def test_centroids_and_scores(dt, d, seq):
    log(f"[select] centroids + scores {dt} d={d} seq={seq}")
    inp = synth.make_inputs(30, 2, 8, 2, d, 64 * 21, dtype=dt, kind="mixture", seq_lens=seq)
    q, k, v, sl = upload(inp)
    import sparse_kv_amd as skv

    C = skv.attn_build_centroids(k, sl)
    sc = skv.attn_score_centroids(q, C, sl)
    torch.cuda.synchronize()
    qf, kf, _ = inp.f64()
    RC = oracle.block_centroids(kf, inp.seq_lens)
    assert_close(C.cpu().numpy(), RC, 1e-5, "centroids")
    RS = oracle.centroid_scores(qf, RC, inp.seq_lens, inp.scale)
    got = sc.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(RS)), "-inf pattern past the end"
    fin = np.isfinite(RS)
    assert_close(got[fin], RS[fin], 1e-4, "scores")


def upload_scores(s):
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).cuda()


@pytest.mark.parametrize("k,ns,nr", [(3, 1, 2), (0, 1, 4), (50, 1, 1), (5, 0, 0), (2, 3, 40), (1, 0, 0)])
def test_topk_exact_on_given_scores(k, ns, nr):
    log(f"[select] top-k k={k} sink={ns} recent={nr}")
    r = np.random.default_rng(k * 100 + ns * 10 + nr)
    B, Hkv, NB = 4, 3, 33
    s = r.standard_normal((B, Hkv, NB)).astype(np.float32)
    s[1, 2, 5:15] = 0.25  # a run of exact ties
    s[2, 0, :] = 1.0  # everything tied
    s[3, 1, 4] = -0.0
    s[3, 1, 9] = 0.0
    seq = np.array([64 * NB, 64 * 10 + 1, 64, 0], dtype=np.int32)
    import sparse_kv_amd as skv

    max_sel = min(NB, ns + nr + k) + 2
    idx, n = skv.attn_select_topk(upload_scores(s) if k > 0 else None, torch.from_numpy(seq).cuda(), k=k,
                                  n_sink_blocks=ns, n_recent_blocks=nr, max_sel=max_sel,
                                  shape=(B, Hkv, NB), device="cuda")
    torch.cuda.synchronize()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    ref = oracle.select_all(s.astype(np.float64), seq, k, ns, nr)
    for b in range(B):
        for g in range(Hkv):
            want = ref[b][g]
            assert n[b, g] == len(want), (b, g, n[b, g], want)
            assert idx[b, g, :len(want)].tolist() == want, (b, g)
            assert (idx[b, g, len(want):] == -1).all()


@pytest.mark.parametrize("NB", [2048, 4096])
def test_topk_large_rows_radix_paths(NB):
    # rows of up to 2048 blocks take the register-resident select, longer rows the LDS-staged one;
    # in both, the 8-bit radix select takes over when the k-th key's 12-bit bin holds over 256 keys
    log(f"[select] top-k on {NB}-block rows")
    r = np.random.default_rng(9)
    B, Hkv = 2, 2
    s = (r.standard_normal((B, Hkv, NB)) * 3).astype(np.float32)
    s[0, 0] = (1.0 + r.integers(0, 3000, NB) * 1e-7).astype(np.float32)  # one 12-bit bin, with ties
    s[0, 1] = np.round(s[0, 1] * 4) / 4  # heavy ties
    s[1, 0, 100:200] = s[1, 0, NB * 3 // 4]  # ties at the boundary region
    s[1, 1, 7] = -0.0
    s[1, 1, 8] = 0.0
    seq = np.array([64 * NB, 64 * (NB * 3 // 4) - 17], dtype=np.int32)
    import sparse_kv_amd as skv

    for k, ns, nr in ((NB // 10, 1, 64), (1, 1, 0), (NB * 3 // 4, 2, 7), (NB, 0, 0), (NB // 2, 0, 0)):
        idx, n = skv.attn_select_topk(upload_scores(s), torch.from_numpy(seq).cuda(), k=k, n_sink_blocks=ns,
                                      n_recent_blocks=nr)
        torch.cuda.synchronize()
        idx, n = idx.cpu().numpy(), n.cpu().numpy()
        ref = oracle.select_all(s.astype(np.float64), seq, k, ns, nr)
        for b in range(B):
            for g in range(Hkv):
                assert idx[b, g, :n[b, g]].tolist() == ref[b][g], (k, b, g)


def margin_inputs(cfg, B, Hq, Hkv, d, L, k, ns, nr, seq=None, **kw):
    """Mixture inputs whose top-k boundary clears a 1e-4 score gap (units redrawn)."""
    attempts = {}
    for _ in range(20):
        inp = synth.make_inputs(cfg, B, Hq, Hkv, d, L, kind="mixture", seq_lens=seq, attempts=attempts, **kw)
        qf, kf, _ = inp.f64()
        sig = oracle.centroid_scores(qf, oracle.block_centroids(kf, inp.seq_lens), inp.seq_lens, inp.scale)
        bad = []
        for b in range(B):
            nb = -(-int(inp.seq_lens[b]) // 64)
            for g in range(Hkv):
                if selection_gap(sig[b, g], nb, k, ns, nr) <= 1e-4:
                    bad.append((b, g))
        if not bad:
            return inp, sig
        for u in bad:
            attempts[u] = attempts.get(u, 0) + 1
    raise AssertionError("could not draw inputs with a selection margin")


def test_selection_pipeline_and_sparse_decode_with_poison():
    log("[select] centroid -> score -> top-k -> sparse decode, unselected blocks poisoned")
    B, Hq, Hkv, d, L = 2, 8, 2, 128, 64 * 200
    k, ns, nr = 20, 1, 6
    inp, sig = margin_inputs(31, B, Hq, Hkv, d, L, k, ns, nr, seq=[64 * 200, 64 * 150 + 30])
    q, kk, v, sl = upload(inp)
    import sparse_kv_amd as skv

    C = skv.attn_build_centroids(kk, sl)
    sc = skv.attn_score_centroids(q, C, sl)
    idx, n = skv.attn_select_topk(sc, sl, k=k, n_sink_blocks=ns, n_recent_blocks=nr)
    torch.cuda.synchronize()
    ref = oracle.select_all(sig, inp.seq_lens, k, ns, nr)
    idx_np, n_np = idx.cpu().numpy(), n.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            assert idx_np[b, g, :n_np[b, g]].tolist() == ref[b][g], (b, g)
    qf, kf, vf = inp.f64()
    want = oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, ref)
    synth.poison_blocks(inp, ref)
    _, kp, vp, _ = upload(inp)
    for S in (1, 3, 8):
        m, l, o = skv.attn_decode_sparse(q, kp, vp, idx, n, sl, num_splits=S)
        out = skv.attn_merge_states(m, l, o)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), want, TOL, f"sparse output S={S}")
    rm, rl, ro = oracle.decode_sparse_split_states(qf, kf, vf, inp.seq_lens, inp.scale, ref, 3)
    m, l, o = skv.attn_decode_sparse(q, kp, vp, idx, n, sl, num_splits=3)
    torch.cuda.synchronize()
    assert_states_close(m, l, o, rm, rl, ro, TOL, "sparse split states")


def test_selecting_everything_equals_dense():
    log("[select] k >= candidates gives dense attention")
    inp = synth.make_inputs(32, 2, 8, 2, 128, 64 * 16, kind="gauss", seq_lens=[64 * 16, 64 * 9 + 1])
    q, k, v, sl = upload(inp)
    import sparse_kv_amd as skv

    sc = skv.attn_score_centroids(q, skv.attn_build_centroids(k, sl), sl)
    idx, n = skv.attn_select_topk(sc, sl, k=100, n_sink_blocks=1, n_recent_blocks=0)
    out = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, sl, num_splits=4))
    dense = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, sl, num_splits=4))
    torch.cuda.synchronize()
    assert n.cpu().tolist() == [[16, 16], [10, 10]]
    assert_close(out.cpu().numpy(), dense.cpu().numpy(), 1e-5, "sparse(all) vs dense")


def test_squeezed_worked_example_on_gpu():
    # Squeezed Attention blog, Q1 worked example, embedded at d = 64 with
    # 64-token blocks: block 0 holds keys like A-C, block 1 keys like D-F.
    log("[select] worked example: the query picks the closer centroid")
    r = np.random.default_rng(2)
    d = 64
    e1, e2 = np.eye(d)[0], np.eye(d)[1]
    K = np.concatenate([e1 * 4 + 0.1 * r.standard_normal((64, d)), e2 * 4 + 0.1 * r.standard_normal((64, d))])
    V = r.standard_normal((128, d))
    qv = e2 * 2 + 0.05 * r.standard_normal(d)
    t = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()
    q, k, v = t(qv[None, None]), t(K[None, None]), t(V[None, None])
    import sparse_kv_amd as skv

    sc = skv.attn_score_centroids(q, skv.attn_build_centroids(k))
    idx, n = skv.attn_select_topk(sc, None, k=1, n_sink_blocks=0, n_recent_blocks=0)
    out = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, None, num_splits=1))
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [[[1]]]
    Kf, Vf, qf = K.astype(np.float32).astype(np.float64), V.astype(np.float32).astype(np.float64), qv.astype(
        np.float32).astype(np.float64)
    want = oracle.decode_blocks(qf[None, None], Kf[None, None], Vf[None, None], np.array([128]), 1 / 8.0, [[[1]]])
    assert_close(out.cpu().numpy(), want, 1e-5, "cluster-2-only output")


@pytest.mark.parametrize("dt,d,hint", [("bf16", 128, 4), ("f32", 64, 1)])
def test_centroid_update_after_appends(dt, d, hint):
    """Centroids built at earlier lengths and refreshed after appends (or a
    shrink) equal the oracle's at the new lengths; blocks before the refreshed
    range are not written."""
    import sparse_kv_amd as skv

    log(f"[select] centroid update {dt} d={d} span_hint={hint}")
    NB = 12
    new = np.array([64 * 12, 64 * 5 + 3, 64 * 7, 40, 64 * 5 + 3, 0], dtype=np.int32)
    old = np.array([64 * 9 + 10, 64 * 5 + 2, 64 * 6, 0, 64 * 8, 0], dtype=np.int32)
    lo = np.minimum(old, new) // 64
    inp = synth.make_inputs(31, 6, 4, 2, d, 64 * NB, dtype=dt, kind="mixture", seq_lens=new)
    q, k, v, sl = upload(inp)
    old_t = torch.from_numpy(old).cuda()
    C = skv.attn_build_centroids(k, old_t)
    for b in range(6):
        C[b, :, :lo[b]] = 123.0  # sentinel: outside the refreshed range
    skv.attn_update_centroids(k, C, sl, prev_lens=old_t, span_hint=hint)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    _, kf, _ = inp.f64()
    ref = oracle.block_centroids(kf, inp.seq_lens)
    for b in range(6):
        assert (got[b, :, :lo[b]] == 123.0).all(), f"row {b}: a block before the range was written"
        assert_close(got[b, :, lo[b]:], ref[b, :, lo[b]:], 1e-5, f"row {b} refreshed blocks")

    log("  one token appended per row, last block only")
    new1 = np.array([64 * 7, 64 * 7 + 1, 1, 64 * 12, 64 * 3 + 30, 65], dtype=np.int32)
    inp = synth.make_inputs(32, 6, 4, 2, d, 64 * NB, dtype=dt, kind="mixture", seq_lens=new1)
    q, k, v, sl = upload(inp)
    C = skv.attn_build_centroids(k, torch.from_numpy(new1 - 1).cuda())
    skv.attn_update_centroids(k, C, sl, span_hint=hint)
    torch.cuda.synchronize()
    _, kf, _ = inp.f64()
    assert_close(C.cpu().numpy(), oracle.block_centroids(kf, inp.seq_lens), 1e-5, "after one-token appends")


@pytest.mark.parametrize("dt,d,group,seq", [("bf16", 128, 4, [64 * 30, 64 * 13 + 5, 0]),
                                           ("f32", 64, 3, [64 * 30, 1, 64 * 7])])
def test_super_centroids(dt, d, group, seq):
    import sparse_kv_amd as skv

    log(f"[select] super-block centroids {dt} d={d} group={group}")
    inp = synth.make_inputs(33, 3, 4, 2, d, 64 * 30, dtype=dt, kind="mixture", seq_lens=seq)
    q, k, v, sl = upload(inp)
    C2 = skv.attn_build_super_centroids(skv.attn_build_centroids(k, sl), group, sl)
    torch.cuda.synchronize()
    _, kf, _ = inp.f64()
    assert_close(C2.cpu().numpy(), oracle.selection.super_centroids(kf, inp.seq_lens, group), 1e-5, "super centroids")


def two_level_inputs(cfg, B, Hq, Hkv, d, L, seq, group, kc, k, ns, nr, dtype="bf16"):
    """Mixture inputs whose two decision boundaries clear 1e-4 (units redrawn)."""
    from oracle.selection import select_all_two_level, super_centroids, two_level_gaps

    attempts = {}
    for _ in range(30):
        inp = synth.make_inputs(cfg, B, Hq, Hkv, d, L, dtype=dtype, kind="mixture", seq_lens=seq, attempts=attempts)
        qf, kf, _ = inp.f64()
        fine = oracle.centroid_scores(qf, oracle.block_centroids(kf, inp.seq_lens), inp.seq_lens, inp.scale)
        coarse = oracle.centroid_scores(qf, super_centroids(kf, inp.seq_lens, group), inp.seq_lens, inp.scale,
                                        block=64 * group)
        bad = []
        for b in range(B):
            nb = -(-int(inp.seq_lens[b]) // 64)
            for g in range(Hkv):
                if min(two_level_gaps(fine[b, g], coarse[b, g], nb, group, kc, k, ns, nr)) <= 1e-4:
                    bad.append((b, g))
        if not bad:
            return inp, select_all_two_level(fine, coarse, inp.seq_lens, group, kc, k, ns, nr)
        for u in bad:
            attempts[u] = attempts.get(u, 0) + 1
    raise AssertionError("could not draw inputs with two-level selection margins")


@pytest.mark.parametrize("label,group,kc,k,ns,nr,seq", [
    ("g4 open 3 of 8", 4, 3, 5, 1, 2, [64 * 32, 64 * 21 + 7]),
    ("g8 open 1", 8, 1, 3, 1, 4, [64 * 32, 64 * 32]),
    ("g3 open all = one level", 3, 100, 7, 1, 1, [64 * 32, 64 * 17]),
    ("g5 forced only", 5, 0, 4, 2, 3, [64 * 32, 64 * 4]),
    ("g4 short rows", 4, 2, 6, 1, 1, [64 * 2 + 1, 0]),
    ("g16 window covers most", 16, 2, 8, 1, 20, [64 * 32, 64 * 25]),
])
def test_two_level_selection_exact(label, group, kc, k, ns, nr, seq):
    import sparse_kv_amd as skv

    log(f"[select] two-level: {label}")
    inp, lists = two_level_inputs(34, 2, 8, 2, 128, 64 * 32, seq, group, kc, k, ns, nr)
    q, kk, v, sl = upload(inp)
    C = skv.attn_build_centroids(kk, sl)
    C2 = skv.attn_build_super_centroids(C, group, sl)
    idx, n = skv.attn_select_two_level(q, C, C2, group, sl, k_coarse=kc, k=k, n_sink_blocks=ns, n_recent_blocks=nr)
    torch.cuda.synchronize()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    for b in range(2):
        for g in range(2):
            assert idx[b, g, :n[b, g]].tolist() == lists[b][g], (b, g)
            assert (idx[b, g, n[b, g]:] == -1).all()
    if kc >= 100:
        one = skv.attn_select_topk(skv.attn_score_centroids(q, C, sl), sl, k=k, n_sink_blocks=ns, n_recent_blocks=nr)
        torch.cuda.synchronize()
        assert np.array_equal(one[0].cpu().numpy(), idx) and np.array_equal(one[1].cpu().numpy(), n)


def test_decoupled_forecast_selection():
    """Selection driven by a per-KV-head forecast vector that is not the
    attention query (one forecast head per GQA group); attention then runs
    with the real queries over the forecast's blocks."""
    import sparse_kv_amd as skv
    from tests.gpu_util import to_dev

    log("[select] decoupled forecast query")
    B, Hq, Hkv, d, L = 2, 8, 2, 128, 64 * 40
    k_top, ns, nr = 6, 1, 3
    attempts = {}
    for _ in range(30):
        inp = synth.make_inputs(35, B, Hq, Hkv, d, L, kind="mixture", seq_lens=[64 * 40, 64 * 27 + 11],
                                attempts=attempts)
        fc = synth.round_to_bf16(np.random.default_rng(3500 + sum(attempts.values())).standard_normal(
            (B, Hkv, d)).astype(np.float32))
        qf, kf, vf = inp.f64()
        ff = synth.bf16_to_f32(fc).astype(np.float64)
        sig = oracle.centroid_scores(ff, oracle.block_centroids(kf, inp.seq_lens), inp.seq_lens, inp.scale)
        bad = [(b, g) for b in range(B) for g in range(Hkv)
               if selection_gap(sig[b, g], -(-int(inp.seq_lens[b]) // 64), k_top, ns, nr) <= 1e-4]
        if not bad:
            break
        for u in bad:
            attempts[u] = attempts.get(u, 0) + 1
    else:
        raise AssertionError("no margin")
    lists = oracle.select_all(sig, inp.seq_lens, k_top, ns, nr)
    q, k, v, sl = upload(inp)
    f = to_dev(fc, "bf16")
    C = skv.attn_build_centroids(k, sl)
    idx, n = skv.attn_select_topk(skv.attn_score_centroids(f, C, sl, scale=inp.scale), sl, k=k_top,
                                  n_sink_blocks=ns, n_recent_blocks=nr)
    out = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, sl, num_splits=3))
    torch.cuda.synchronize()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            assert idx[b, g, :n[b, g]].tolist() == lists[b][g]
    assert_close(out.cpu().numpy(), oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, lists), TOL,
                 "attention over the forecast's blocks")
