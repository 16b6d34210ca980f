"""Pins of the ART oracle (CPU only)."""

import math

import numpy as np
import pytest

import oracle
from oracle.art import art_decode, art_decode_head, art_margin_ok, default_order, probe_metrics
from tests import brute


def inputs(seed, L=80, d=16, block=8):
    r = np.random.default_rng(seed)
    q = r.standard_normal((1, 2, d))
    k = r.standard_normal((1, 1, L, d)) * 1.5
    v = r.standard_normal((1, 1, L, d))
    return q, k, v, np.array([L])


def test_default_order():
    assert default_order(1) == [0]
    assert default_order(5) == [0, 4, 3, 2, 1]
    assert default_order(0) == []


def test_probe_metrics_closed_forms():
    for theta in (0.0, 0.01, 0.3, 1.0, math.pi / 2, 3.0):
        x = np.array([1.0, 0.0, 0.0])
        y = np.array([math.cos(theta), math.sin(theta), 0.0]) * 2.5
        ds, dd = probe_metrics(y, x)
        assert abs(ds - 1.5) < 1e-15
        assert abs(dd - (1 - math.cos(theta))) < 1e-15
    # zero norm is never stable
    ds, dd = probe_metrics(np.zeros(3), np.array([1.0, 0, 0]))
    assert ds == 1.0 and dd == math.inf
    assert not oracle.art.is_stable(0.0, dd, 1.0, 1.0)


def test_zero_thresholds_give_dense():
    q, k, v, seq = inputs(0)
    dense = oracle.decode_dense(q, k, v, seq, 0.25, block=8)
    out, stop, _ = art_decode(q, k, v, seq, 0.25, 0.0, 0.0, 1, 8, block=8)
    assert (stop == 9).all() and np.max(np.abs(out - dense)) < 1e-12
    # any order starting with block 0 gives the same dense output
    order = [[[0] + list(np.random.default_rng(3).permutation(np.arange(1, 10)))]]
    out2, stop2, _ = art_decode(q, k, v, seq, 0.25, 0.0, 0.0, 1, 8, order=order, block=8)
    assert (stop2 == 9).all() and np.max(np.abs(out2 - dense)) < 1e-12


def test_patience_longer_than_sequence_and_detector_off():
    q, k, v, seq = inputs(1)
    dense = oracle.decode_dense(q, k, v, seq, 0.25, block=8)
    out, stop, _ = art_decode(q, k, v, seq, 0.25, math.inf, math.inf, 11, 8, block=8)
    assert (stop == 9).all() and np.max(np.abs(out - dense)) < 1e-12
    out, stop, tr = art_decode(q, k, v, seq, 0.25, math.inf, math.inf, 1, 0, block=8)
    assert (stop == 9).all() and tr[(0, 0)] == []


def test_infinite_thresholds_stop_after_second_block():
    q, k, v, seq = inputs(2)
    out, stop, _ = art_decode(q, k, v, seq, 0.25, math.inf, math.inf, 1, 8, block=8)
    assert (stop == 1).all()
    # attention over blocks pi_0 = 0 and pi_1 = nb - 1 = 9
    toks = list(range(0, 8)) + list(range(72, 80))
    for h in range(2):
        ref = brute.attention_over_tokens(list(q[0, h]), k[0, 0], v[0, 0], toks, 0.25)
        assert np.max(np.abs(out[0, h] - np.array(ref))) < 1e-12


@pytest.mark.parametrize("j,p", [(1, 1), (3, 2), (4, 3), (2, 1)])
def test_constant_probe_construction_stops_at_j_plus_p(j, p):
    # If every value row visited after position j equals O_j, the partial
    # output stops moving: d = 0 from step j+1 on, so the stop is exactly j+p.
    q, k, v, seq = inputs(4 + j)
    scale = 0.25
    nb, blk = 10, 8
    order = default_order(nb)
    h = 0
    O_j = art_decode_head(q[0, h], k[0, 0], v[0, 0], 80, scale, order[:j + 1], 0, 0, 1, 8, blk)[0]
    v2 = v.copy()
    for jj in order[j + 1:]:
        v2[0, 0, jj * blk:(jj + 1) * blk] = O_j
    O, T, trace = art_decode_head(q[0, h], k[0, 0], v2[0, 0], 80, scale, order, 1e-6, 1e-9, p, 8, blk)
    steps = {t: st for t, _, _, st, _ in trace}
    assert steps[j] is False or j == 0  # the change at step j itself is large
    assert T == j + p
    assert np.max(np.abs(O - O_j)) < 1e-12


def test_per_head_stops_differ_under_gqa():
    # head 0 sees flat attention (large changes keep going), head 1 a dominant sink
    q, k, v, seq = inputs(8)
    k[0, 0, :8] = 0.0
    q[0, 1] = 0.0
    q[0, 1, 0] = 30.0
    k[0, 0, :8, 0] = 5.0  # head 1 attends almost only to block 0
    out, stop, traces = art_decode(q, k, v, seq, 0.25, 1e-3, 1e-4, 2, 8, block=8)
    assert stop[0, 1] == 2  # stable from step 1 on
    assert stop[0, 0] > stop[0, 1]


def test_margin_helper():
    tr = [(1, 5e-3, 1e-3, False, 0), (2, 5e-4, 5e-5, True, 1)]
    assert art_margin_ok(tr, 1e-3, 1e-4)
    assert not art_margin_ok([(1, 0.995e-3, 5e-5, True, 1)], 1e-3, 1e-4)
    assert not art_margin_ok([(1, 1.005e-3, 5e-5, False, 0)], 1e-3, 1e-4)


def test_importance_order():
    s = np.array([9.0, 1.0, 3.0, 3.0, -2.0, 7.0, 3.0])
    # block 0 first whatever its score, then descending score, ties to the lower index
    assert oracle.importance_order(s, 7) == [0, 5, 2, 3, 6, 1, 4]
    assert oracle.importance_order(s, 1) == [0]
    assert oracle.importance_order(s, 0) == []
    r = np.random.default_rng(4)
    x = r.standard_normal(50)
    o = oracle.importance_order(x, 50)
    assert o[0] == 0 and sorted(o) == list(range(50))
    assert all(np.float32(x[a]) >= np.float32(x[b]) for a, b in zip(o[1:], o[2:]))


def test_art_over_a_listed_subset():
    # visiting only listed blocks: with tau = phi = 0 it is attention over those blocks
    q, k, v, seq = inputs(6)
    lst = [0, 7, 3, 9]
    out, stop, _ = art_decode(q, k, v, seq, 0.25, 0.0, 0.0, 1, 8, order=[[lst]], n_visit=[[4]], block=8)
    assert (stop == 3).all()
    ref = oracle.decode_blocks(q, k, v, seq, 0.25, [[sorted(lst)]], block=8)
    assert np.max(np.abs(out - ref)) < 1e-12
    # n_visit = 0 visits nothing
    out, stop, _ = art_decode(q, k, v, seq, 0.25, 0.0, 0.0, 1, 8, order=[[lst]], n_visit=[[0]], block=8)
    assert (stop == -1).all() and not out.any()
    # a stop inside the list: tau = phi = inf, p = 1 stops at the second listed block
    out, stop, _ = art_decode(q, k, v, seq, 0.25, math.inf, math.inf, 1, 8, order=[[lst]], n_visit=[[4]], block=8)
    assert (stop == 1).all()
    toks = list(range(0, 8)) + list(range(56, 64))
    ref = brute.attention_over_tokens(list(q[0, 0]), k[0, 0], v[0, 0], toks, 0.25)
    assert np.max(np.abs(out[0, 0] - np.array(ref))) < 1e-12
