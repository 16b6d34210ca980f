"""GPU parity: importance-first visit order, and ART over listed blocks."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.art import art_margin_ok
from oracle.selection import selection_gap
from tests.gpu_util import TOL, assert_close, log, upload

pytestmark = pytest.mark.gpu

TAU, PHI, P, PROBE = 1e-3, 1e-4, 2, 8


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def oracle_scores_f32(inp):
    """Centroid scores by the oracle, rounded to the float32 the order is taken in."""
    qf, kf, _ = inp.f64()
    cent = oracle.block_centroids(kf, inp.seq_lens)
    return oracle.centroid_scores(qf, cent, inp.seq_lens, inp.scale).astype(np.float32)


def expected_order(scores, seq_lens, NBmax):
    B, Hkv, _ = scores.shape
    ref = np.full((B, Hkv, NBmax), -1, dtype=np.int32)
    for b in range(B):
        nb = -(-int(seq_lens[b]) // 64)
        for g in range(Hkv):
            o = oracle.importance_order(scores[b, g], nb)
            ref[b, g, :len(o)] = o
    return ref


@pytest.mark.parametrize("label,B,Hkv,NBmax,seq", [
    ("ragged-100", 3, 2, 100, [64 * 100, 64 * 37 + 5, 0]),
    ("tiny rows", 4, 1, 3, [1, 64, 65, 64 * 3]),
    ("4097 blocks", 1, 2, 4097, None),
    ("4098 blocks (large table)", 1, 1, 4098, None),
    ("16385 blocks (maximum)", 1, 1, 16385, None),
])
def test_order_blocks_exact(label, B, Hkv, NBmax, seq):
    import sparse_kv_amd as skv

    log(f"[order] {label}")
    r = np.random.default_rng(NBmax)
    sc = r.standard_normal((B, Hkv, NBmax)).astype(np.float32)
    # planted ties: repeated values, and -0 against +0
    sc[..., 5::7] = np.float32(0.5)
    if NBmax > 12:
        sc[..., 10] = np.float32(-0.0)
        sc[..., 11] = np.float32(0.0)
        sc[..., 12] = np.float32(0.0)
    seq_lens = np.full(B, NBmax * 64, dtype=np.int32) if seq is None else np.array(seq, dtype=np.int32)
    got = skv.attn_order_blocks(torch.from_numpy(sc).cuda(), dev_i32(seq_lens)).cpu().numpy()
    ref = expected_order(sc, seq_lens, NBmax)
    assert np.array_equal(got, ref), f"{label}: first mismatch at {np.argwhere(got != ref)[:3].tolist()}"


def test_order_blocks_from_oracle_centroid_scores():
    import sparse_kv_amd as skv

    log("[order] oracle centroid scores of mixture keys, ragged")
    inp = synth.make_inputs(50, 2, 8, 2, 128, 64 * 60, kind="mixture", seq_lens=[64 * 60, 64 * 23 + 9])
    sc = oracle_scores_f32(inp)
    got = skv.attn_order_blocks(torch.from_numpy(sc).cuda(), dev_i32(inp.seq_lens)).cpu().numpy()
    assert np.array_equal(got, expected_order(sc, inp.seq_lens, 60))


def margin_inputs(cfg, B, Hq, Hkv, d, L, seq=None, kind="recency", recent=64 * 6):
    """Inputs whose importance order is clear (sorted float32 oracle scores
    1e-4 apart) and whose every ART decision in that order clears a 1% band."""
    attempts = {}
    G = Hq // Hkv
    for _ in range(30):
        inp = synth.make_inputs(cfg, B, Hq, Hkv, d, L, kind=kind, seq_lens=seq, attempts=attempts,
                                recent_tokens=recent)
        qf, kf, vf = inp.f64()
        sc = oracle.centroid_scores(qf, oracle.block_centroids(kf, inp.seq_lens), inp.seq_lens, inp.scale)
        NBmax = L // 64
        order = expected_order(sc.astype(np.float32), inp.seq_lens, NBmax)
        bad = set()
        for b in range(B):
            nb = -(-int(inp.seq_lens[b]) // 64)
            for g in range(Hkv):
                s = sc[b, g, order[b, g, 1:nb]]
                if nb > 2 and np.min(s[:-1] - s[1:]) <= 1e-4:
                    bad.add((b, g))
        out, stop, traces = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, TAU, PHI, P, PROBE,
                                              order=order)
        bad |= {(b, h // G) for (b, h), tr in traces.items() if not art_margin_ok(tr, TAU, PHI)}
        if not bad:
            return inp, order, out, stop
        for u in bad:
            attempts[u] = attempts.get(u, 0) + 1
    raise AssertionError("could not draw inputs with order and ART margins")


@pytest.mark.parametrize("label,B,Hq,Hkv,d,L,seq,kind", [
    ("recency bf16 g4", 2, 8, 2, 128, 64 * 40, [64 * 40, 64 * 29 + 3], "recency"),
    ("mixture bf16 g4 d64", 1, 8, 2, 64, 64 * 32, None, "mixture"),
])
def test_importance_first_art_end_to_end(label, B, Hq, Hkv, d, L, seq, kind):
    """Centroids -> scores -> order -> ART on the GPU against the oracle's own chain."""
    import sparse_kv_amd as skv

    log(f"[order] importance-first ART: {label}")
    inp, ref_order, ref_out, ref_stop = margin_inputs(60, B, Hq, Hkv, d, L, seq=seq, kind=kind)
    q, k, v, sl = upload(inp)
    order = skv.attn_order_blocks(skv.attn_score_centroids(q, skv.attn_build_centroids(k, sl), sl), sl)
    out, stop, fetched = skv.attn_decode_art(q, k, v, sl, order=order, tau=TAU, phi=PHI, patience=P,
                                             probe_dim=PROBE)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), ref_order)
    stop = stop.cpu().numpy()
    log(f"  stops {ref_stop.ravel().tolist()}")
    assert np.array_equal(stop, ref_stop)
    assert_close(out.cpu().numpy(), ref_out, TOL, "importance-first ART output")


def art_list(path):
    import sparse_kv_amd as skv

    return skv.attn_decode_art_list_ws if path == "ws" else skv.attn_decode_art_list


def list_case(cfg, B, Hq, Hkv, d, L, seq, kind, k, ns, nr, max_list, newest_first=False, require_inside=False,
              recent=64 * 5):
    """Inputs and block lists for ART over a selection: per unit the oracle's top-k list
    (ascending, so block 0 first), or block 0 then the other listed blocks newest first.
    Units are redrawn until every top-k boundary gap exceeds 1e-4, every thresholded ART
    decision clears the 1% band and, with require_inside, every head stops strictly
    inside its list.  Returns (inputs, lists, block_list, n_list)."""
    attempts = {}
    G = Hq // Hkv
    for _ in range(40):
        inp = synth.make_inputs(cfg, B, Hq, Hkv, d, L, kind=kind, seq_lens=seq, attempts=attempts,
                                recent_tokens=recent)
        qf, kf, vf = inp.f64()
        sc = oracle.centroid_scores(qf, oracle.block_centroids(kf, inp.seq_lens), inp.seq_lens, inp.scale)
        lists = oracle.select_all(sc, inp.seq_lens, k, ns, nr)
        bl = np.full((B, Hkv, max_list), -1, dtype=np.int32)
        nl = np.zeros((B, Hkv), dtype=np.int32)
        bad = set()
        for b in range(B):
            nb = -(-int(inp.seq_lens[b]) // 64)
            for g in range(Hkv):
                x = lists[b][g]
                if newest_first:
                    x = x[:1] + sorted(x[1:], reverse=True)
                bl[b, g, :len(x)] = x
                nl[b, g] = len(x)
                if not selection_gap(sc[b, g], nb, k, ns, nr) > 1e-4:
                    bad.add((b, g))
        _, stop, traces = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, TAU, PHI, P, PROBE, order=bl,
                                            n_visit=nl)
        bad |= {(b, h // G) for (b, h), tr in traces.items() if not art_margin_ok(tr, TAU, PHI)}
        if require_inside:
            bad |= {(b, h // G) for b in range(B) for h in range(Hq) if not stop[b, h] < nl[b, h // G] - 1}
        if not bad:
            return inp, lists, bl, nl
        for u in bad:
            attempts[u] = attempts.get(u, 0) + 1
    raise AssertionError("could not draw list inputs with selection and ART decision margins")


def run_art_list(path, inp, lists, bl, nl, tau, phi, p):
    """ART over the lists on a copy of the cache whose unlisted blocks hold NaN."""
    poisoned = synth.DecodeInputs(inp.q, inp.k.copy(), inp.v.copy(), inp.seq_lens, inp.dtype)
    synth.poison_blocks(poisoned, lists)
    q, k, v, sl = upload(poisoned)
    out, stop, fetched = art_list(path)(q, k, v, dev_i32(bl), dev_i32(nl), sl, tau=tau, phi=phi, patience=p,
                                        probe_dim=PROBE)
    torch.cuda.synchronize()
    return out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()


@pytest.mark.parametrize("path", ["one", "ws"])
def test_art_over_selected_lists(path):
    """attn_decode_art_list[_ws] on the oracle's top-k lists; unlisted blocks hold NaN."""
    log(f"[order] ART over top-k lists (sink first, ascending), {path}")
    B, Hq, Hkv, d, L = 2, 8, 2, 128, 64 * 48
    inp, lists, bl, nl = list_case(61, B, Hq, Hkv, d, L, [64 * 48, 64 * 31 + 20], "recency", 12, 1, 4, 20)
    qf, kf, vf = inp.f64()
    for tau, phi, p in ((TAU, PHI, P), (0.0, 0.0, 1), (math.inf, math.inf, 1)):
        ref_out, ref_stop, _ = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, tau, phi, p, PROBE,
                                                 order=bl, n_visit=nl)
        out, stop, fetched = run_art_list(path, inp, lists, bl, nl, tau, phi, p)
        log(f"  tau={tau}: stops {stop.ravel().tolist()}")
        assert np.array_equal(stop, ref_stop)
        assert_close(out, ref_out, TOL, f"ART over lists tau={tau}")
        assert (fetched <= nl).all()
        if tau == 0.0:
            assert (stop == nl.repeat(Hq // Hkv, axis=1) - 1).all()
            dense_lists = oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale,
                                               [[sorted(x) for x in row] for row in lists])
            assert_close(out, dense_lists, TOL, "tau = 0 equals attention over the lists")
        if tau == math.inf:
            assert (stop == 1).all()


@pytest.mark.parametrize("path", ["one", "ws"])
@pytest.mark.parametrize("label,cfg,L,seq,kind,k,nr,newest_first", [
    ("recency keys, newest listed block first, 17 listed", 63, 64 * 48, [64 * 48, 64 * 37 + 20], "recency", 12, 4,
     True),
    ("mixture keys, ascending lists, 89 listed", 64, 64 * 400, [64 * 400, 64 * 350 - 7], "mixture", 80, 8, False),
])
def test_art_over_lists_stops_inside_the_list(label, cfg, L, seq, kind, k, nr, newest_first, path):
    """Finite thresholds (tau 1e-3, phi 1e-4, p 2) stop every head strictly inside its list
    ("ART" summary §2.4: the stop rule as a control layer over a selection); stops exact,
    outputs within tolerance, unlisted blocks NaN, read-ahead within the list."""
    log(f"[order] ART over lists, stop inside: {label}, {path}")
    B, Hq, Hkv, d = 2, 8, 2, 128
    inp, lists, bl, nl = list_case(cfg, B, Hq, Hkv, d, L, seq, kind, k, 1, nr, k + 1 + nr + 3,
                                   newest_first=newest_first, require_inside=True)
    qf, kf, vf = inp.f64()
    ref_out, ref_stop, _ = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, TAU, PHI, P, PROBE, order=bl,
                                             n_visit=nl)
    assert (ref_stop < nl.repeat(Hq // Hkv, axis=1) - 1).all()
    out, stop, fetched = run_art_list(path, inp, lists, bl, nl, TAU, PHI, P)
    log(f"  lists of {nl.ravel().tolist()}: stops {stop.ravel().tolist()}, fetched {fetched.ravel().tolist()}")
    assert np.array_equal(stop, ref_stop)
    assert_close(out, ref_out, TOL, "ART over lists, stopped inside")
    need = stop.reshape(B, Hkv, -1).max(axis=2) + 1
    assert (need <= fetched).all() and (fetched <= nl).all()


@pytest.mark.parametrize("path", ["one", "ws"])
def test_art_list_edge_counts(path):
    """n_list = 0, n_list past the sequence and past max_list, ragged rows."""
    log(f"[order] ART list edge counts, {path}")
    B, Hq, Hkv, d, L = 3, 4, 1, 128, 64 * 10
    inp = synth.make_inputs(62, B, Hq, Hkv, d, L, kind="gauss", seq_lens=[64 * 10, 64 * 3 + 1, 64 * 10])
    max_list = 6
    bl = np.array([[[0, 9, 2, 5, 7, 1]], [[0, 3, 1, 2, -1, -1]], [[0, 4, 8, 3, 6, 2]]], dtype=np.int32)
    nl = np.array([[0], [9], [100]], dtype=np.int32)  # 0 -> nothing; 9 -> nb = 4; 100 -> max_list = 6
    q, k, v, sl = upload(inp)
    out, stop, fetched = art_list(path)(q, k, v, dev_i32(bl), dev_i32(nl), sl, tau=0.0, phi=0.0, patience=1,
                                        probe_dim=PROBE)
    torch.cuda.synchronize()
    out, stop, fetched = out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()
    assert stop[0].tolist() == [-1] * Hq and not out[0].any() and fetched[0, 0] == 0
    assert stop[1].tolist() == [3] * Hq and fetched[1, 0] == 4
    assert stop[2].tolist() == [5] * Hq and fetched[2, 0] == 6
    qf, kf, vf = inp.f64()
    eff = np.array([[0], [4], [6]])
    ref_out, ref_stop, _ = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, 0.0, 0.0, 1, PROBE,
                                             order=bl, n_visit=eff)
    assert np.array_equal(stop, ref_stop)
    assert_close(out, ref_out, TOL, "edge-count ART")
