"""Pins of the centroid / score / top-k oracle (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.selection import block_centroids, centroid_scores, select_blocks, selection_gap
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_centroids_are_block_means():
    r = np.random.default_rng(0)
    k = r.standard_normal((2, 2, 21, 5))
    seq = np.array([21, 10])
    C = block_centroids(k, seq, block=4)
    assert C.shape == (2, 2, 6, 5)
    for b in range(2):
        L = int(seq[b])
        for g in range(2):
            for j in range(6):
                toks = list(range(j * 4, min(j * 4 + 4, L)))
                if toks:
                    ref = brute.mean_rows([list(k[b, g, t]) for t in toks])
                    assert np.max(np.abs(C[b, g, j] - np.array(ref))) < 1e-15
                else:
                    assert not C[b, g, j].any()


def test_score_is_mean_logit_of_block():
    # <sum_h q_h, c_j> = mean over the block's tokens of <sum_h q_h, k_t> (linearity)
    r = np.random.default_rng(1)
    B, Hq, Hkv, d, L = 1, 4, 2, 6, 19
    q = r.standard_normal((B, Hq, d))
    k = r.standard_normal((B, Hkv, L, d))
    seq = np.array([L])
    sig = centroid_scores(q, block_centroids(k, seq, block=4), seq, 0.5, block=4)
    for g in range(Hkv):
        qsum = [sum(q[0, h, i] for h in range(g * 2, g * 2 + 2)) for i in range(d)]
        for j in range(5):
            toks = range(j * 4, min(j * 4 + 4, L))
            ref = sum(0.5 * brute.dot(qsum, list(k[0, g, t])) for t in toks) / len(toks)
            assert abs(sig[0, g, j] - ref) < 1e-13
    assert np.all(np.isneginf(sig[0, :, 5:]))


def brute_select(scores, nb, k, n_sink, n_recent):
    forced = [j for j in range(nb) if j < n_sink or j >= nb - n_recent]
    cand = [j for j in range(nb) if j not in forced]
    ranked = sorted(cand, key=lambda j: (-float(np.float32(scores[j])), j))
    return sorted(forced + ranked[:k])


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_brute_force(seed):
    r = np.random.default_rng(seed)
    nb = int(r.integers(1, 60))
    scores = r.standard_normal(nb)
    k = int(r.integers(0, nb + 3))
    ns, nr = int(r.integers(0, 3)), int(r.integers(0, 6))
    assert select_blocks(scores, nb, k, ns, nr) == brute_select(scores, nb, k, ns, nr)


def test_select_ties_and_edges():
    s = np.array([0.0, 1.0, 3.0, 1.0, 3.0, 2.0, 1.0, 0.5])
    # ties on 3.0 and on 1.0 go to the lower index
    assert select_blocks(s, 8, 2, 0, 0) == [2, 4]
    assert select_blocks(s, 8, 4, 0, 0) == [1, 2, 4, 5]
    # forced sink and window do not use k slots
    assert select_blocks(s, 8, 1, 1, 2) == [0, 2, 6, 7]
    # k >= |candidates| selects everything; k = 0 keeps only forced blocks
    assert select_blocks(s, 8, 50, 1, 2) == list(range(8))
    assert select_blocks(s, 8, 0, 1, 3) == [0, 5, 6, 7]
    # window and sink overlapping / larger than the sequence
    assert select_blocks(s, 3, 5, 2, 5) == [0, 1, 2]
    assert select_blocks(s, 0, 5, 1, 1) == []
    # gap helper
    assert selection_gap(s, 8, 1, 0, 0) == 0.0
    assert selection_gap(np.array([5.0, 4.0, 1.0]), 3, 1, 0, 0) == 1.0


def test_select_all_blocks_gives_dense():
    r = np.random.default_rng(7)
    q = r.standard_normal((1, 2, 8))
    k = r.standard_normal((1, 1, 50, 8))
    v = r.standard_normal((1, 1, 50, 8))
    seq = np.array([50])
    sig = centroid_scores(q, block_centroids(k, seq, block=8), seq, 0.3, block=8)
    lists = oracle.select_all(sig, seq, 100, 1, 1, block=8)
    assert lists[0][0] == list(range(7))
    a = oracle.decode_blocks(q, k, v, seq, 0.3, lists, block=8)
    assert np.max(np.abs(a - oracle.decode_dense(q, k, v, seq, 0.3, block=8))) < 1e-13


def test_squeezed_worked_example():
    # Squeezed Attention blog, Q1 worked example (fixture cites it).
    g = json.load(open(os.path.join(GOLDEN, "squeezed_toy.json")))
    K = np.array(g["keys"])[None, None]
    V = np.array(g["values"])[None, None]
    q = np.array(g["query"])[None, None]
    bs = g["block_size"]
    seq = np.array([K.shape[2]])
    scale = 1 / math.sqrt(K.shape[-1])
    sig = centroid_scores(q, block_centroids(K, seq, block=bs), seq, scale, block=bs)
    lists = oracle.select_all(sig, seq, 1, 0, 0, block=bs)
    assert lists[0][0] == g["expected_selected_blocks"]
    chosen = [g["key_names"].index(n) for n in g["expected_attended_keys"]]
    out = oracle.decode_blocks(q, K, V, seq, scale, lists, block=bs)
    ref = brute.attention_over_tokens(list(q[0, 0]), K[0, 0], V[0, 0], chosen, scale)
    assert np.max(np.abs(out[0, 0] - np.array(ref))) < 1e-14
    # and it differs from full attention (the other cluster is really dropped)
    assert np.max(np.abs(out - oracle.decode_dense(q, K, V, seq, scale, block=bs))) > 1e-3


# ---- two-level (super-block) selection -------------------------------------

from oracle.selection import select_blocks_two_level, super_centroids, two_level_gaps  # noqa: E402


def test_super_centroids_are_means_of_their_tokens():
    r = np.random.default_rng(11)
    k = r.standard_normal((2, 1, 30, 4))
    seq = np.array([30, 13])
    C2 = super_centroids(k, seq, group=2, block=4)  # super-blocks of 8 tokens
    assert C2.shape == (2, 1, 4, 4)
    for b in range(2):
        L = int(seq[b])
        for s_ in range(4):
            toks = list(range(8 * s_, min(8 * s_ + 8, L)))
            if toks:
                ref = brute.mean_rows([list(k[b, 0, t]) for t in toks])
                assert np.max(np.abs(C2[b, 0, s_] - np.array(ref))) < 1e-15
            else:
                assert not C2[b, 0, s_].any()
    # the coarse score is the mean logit of the super-block's tokens (linearity)
    q = r.standard_normal((2, 2, 4))
    sig2 = centroid_scores(q, C2, np.array([4, 2]), 0.7, block=1)  # lengths in super-blocks
    for b in range(2):
        L = int(seq[b])
        qsum = [q[b, 0, i] + q[b, 1, i] for i in range(4)]
        for s_ in range(-(-L // 8)):
            toks = range(8 * s_, min(8 * s_ + 8, L))
            ref = sum(0.7 * brute.dot(qsum, list(k[b, 0, t])) for t in toks) / len(toks)
            assert abs(sig2[b, 0, s_] - ref) < 1e-13


@pytest.mark.parametrize("seed", range(8))
def test_two_level_reduces_to_one_level(seed):
    r = np.random.default_rng(100 + seed)
    nb = int(r.integers(1, 70))
    group = int(r.integers(1, 9))
    fine = r.standard_normal(nb)
    coarse = r.standard_normal(-(-nb // group))
    k = int(r.integers(0, nb + 2))
    ns, nr = int(r.integers(0, 3)), int(r.integers(0, 8))
    # every super-block opened: the one-level choice
    assert select_blocks_two_level(fine, coarse, nb, group, 10 ** 6, k, ns, nr) == select_blocks(fine, nb, k, ns, nr)
    # group = 1 with coarse = fine: the one-level choice with min(k, k_coarse) picks
    kc = int(r.integers(0, nb + 2))
    assert select_blocks_two_level(fine, fine, nb, 1, kc, k, ns, nr) == select_blocks(fine, nb, min(k, kc), ns, nr)


def test_two_level_coarse_gate():
    # 3 super-blocks of 4 blocks.  Super-block 1 has the best mean, super-block
    # 2 holds the single best block.  One-level top-2 takes block 9 (in super-
    # block 2); two-level with one opened super-block stays inside super-block 1.
    fine = np.array([0.0, 0.1, 0.2, 0.3, 2.0, 2.5, 2.2, 2.1, -1.0, 9.0, -1.0, -1.0])
    coarse = np.array([0.15, 2.2, 1.5])
    assert select_blocks(fine, 12, 2, 0, 0) == [5, 9]
    assert select_blocks_two_level(fine, coarse, 12, 4, 1, 2, 0, 0) == [5, 6]
    assert select_blocks_two_level(fine, coarse, 12, 4, 2, 2, 0, 0) == [5, 9]
    # forced sink and window: super-block 0 keeps candidates 1-3, super-block 2
    # none once the window covers blocks 8-11, so it cannot be opened
    assert select_blocks_two_level(fine, coarse, 12, 4, 1, 2, 1, 4) == [0, 5, 6, 8, 9, 10, 11]
    assert select_blocks_two_level(fine, coarse, 12, 4, 2, 5, 1, 4) == [0, 3, 4, 5, 6, 7, 8, 9, 10, 11]
    # ties: the lower super-block and the lower block win
    assert select_blocks_two_level(np.ones(8), np.ones(2), 8, 4, 1, 2, 0, 0) == [0, 1]
    # k_coarse = 0 or k = 0 keep only forced blocks; an empty sequence selects nothing
    assert select_blocks_two_level(fine, coarse, 12, 4, 0, 5, 1, 1) == [0, 11]
    assert select_blocks_two_level(fine, coarse, 12, 4, 3, 0, 1, 1) == [0, 11]
    assert select_blocks_two_level(fine, coarse, 0, 4, 3, 3, 1, 1) == []
    # the gap helper sees both boundaries
    cg, fg = two_level_gaps(fine, coarse, 12, 4, 1, 2, 0, 0)
    assert abs(cg - 0.7) < 1e-12 and abs(fg - 0.1) < 1e-12
