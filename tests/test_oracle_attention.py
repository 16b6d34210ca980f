"""Pins of the dense / split / merge oracle (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import decode_dense, decode_split_states, head_state, merge_state_arrays, merge_states
from tests import brute


def rand_inputs(seed, B=2, Hq=4, Hkv=2, d=8, L=40, ragged=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, d))
    k = r.standard_normal((B, Hkv, L, d)) * 1.5
    v = r.standard_normal((B, Hkv, L, d))
    seq = np.array([L] * B)
    if ragged and B > 1:
        seq[0] = L - 13
    return q, k, v, seq


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_matches_pure_python(seed):
    q, k, v, seq = rand_inputs(seed)
    scale = 1 / math.sqrt(q.shape[-1])
    out = decode_dense(q, k, v, seq, scale, block=8)
    G = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            ref = brute.attention_over_tokens(list(q[b, h]), k[b, h // G], v[b, h // G],
                                              range(int(seq[b])), scale)
            assert np.max(np.abs(out[b, h] - np.array(ref))) < 1e-12


def test_gqa_mapping_uses_consecutive_heads():
    # KV heads made very different: a wrong head -> group map fails loudly.
    q, k, v, seq = rand_inputs(5, B=1, Hq=6, Hkv=3, L=16, ragged=False)
    v[0, 1] += 10.0
    out = decode_dense(q, k, v, seq, 0.3, block=8)
    assert np.all(out[0, 2:4].mean(axis=-1) > 5) and np.all(np.abs(out[0, [0, 1, 4, 5]].mean(axis=-1)) < 5)


def test_dense_matches_torch_softmax_f64():
    q, k, v, seq = rand_inputs(3, B=1, Hq=2, Hkv=1, d=16, L=70, ragged=False)
    scale = 0.25
    out = decode_dense(q, k, v, seq, scale)
    K = torch.from_numpy(k[0, 0])
    V = torch.from_numpy(v[0, 0])
    for h in range(2):
        p = torch.softmax(scale * (K @ torch.from_numpy(q[0, h])), dim=0)
        assert np.max(np.abs(out[0, h] - (p @ V).numpy())) < 1e-13


def test_closed_forms():
    r = np.random.default_rng(9)
    q = r.standard_normal(8)
    V = r.standard_normal((5, 8))
    # a single token returns its value row
    m, l, O = head_state(q, r.standard_normal((1, 8)), V[:1], 0.5)
    assert l == 1.0 and np.allclose(O, V[0], atol=0, rtol=0)
    # identical keys give the mean of the values
    K = np.tile(r.standard_normal(8), (5, 1))
    _, l, O = head_state(q, K, V, 0.5)
    assert abs(l - 5.0) < 1e-12 and np.max(np.abs(O - V.mean(axis=0))) < 1e-14
    # empty set
    m, l, O = head_state(q, np.zeros((0, 8)), np.zeros((0, 8)), 0.5)
    assert m == -math.inf and l == 0.0 and not O.any()


@pytest.mark.parametrize("seed", range(4))
def test_split_merge_equals_unsplit(seed):
    r = np.random.default_rng(100 + seed)
    n, d = 37, 6
    q = r.standard_normal(d)
    K = r.standard_normal((n, d)) * 2
    V = r.standard_normal((n, d))
    whole = head_state(q, K, V, 0.7)
    perm = r.permutation(n)
    cuts = sorted(r.choice(np.arange(1, n), size=4, replace=False))
    parts = np.split(perm, cuts)
    parts.append(np.array([], dtype=int))  # an empty part
    states = [head_state(q, K[p], V[p], 0.7) for p in parts]
    M, Ls, O = merge_states(states, d)
    assert abs(M - whole[0]) < 1e-12 and abs(Ls - whole[1]) < 1e-9 * whole[1]
    assert np.max(np.abs(O - whole[2])) < 1e-12
    # associativity and the empty-state identity
    a, b, c = states[0], states[1], states[2]
    left = merge_states([merge_states([a, b], d), c], d)
    right = merge_states([a, merge_states([b, c], d)], d)
    assert np.max(np.abs(left[2] - right[2])) < 1e-13
    same = merge_states([a, (-math.inf, 0.0, np.zeros(d))], d)
    assert same[0] == a[0] and same[1] == a[1] and np.array_equal(same[2], a[2])
    empty = merge_states([(-math.inf, 0.0, np.zeros(d))] * 3, d)
    assert empty[0] == -math.inf and empty[1] == 0.0 and not empty[2].any()


@pytest.mark.parametrize("S", [1, 3, 5, 16])
def test_split_states_merge_to_dense(S):
    q, k, v, seq = rand_inputs(11, B=2, Hq=4, Hkv=2, d=8, L=40)
    scale = 0.35
    m, l, o = decode_split_states(q, k, v, seq, scale, S, block=8)
    O, M, Ls = merge_state_arrays(m, l, o)
    ref = decode_dense(q, k, v, seq, scale, block=8)
    assert np.max(np.abs(O - ref)) < 1e-12
    # split s holds blocks [floor(s*nb/S), floor((s+1)*nb/S)) -- check one split by brute force
    b, h, s = 0, 1, S - 1
    nb = -(-int(seq[b]) // 8)
    lo, hi = (s * nb) // S, ((s + 1) * nb) // S
    toks = range(lo * 8, min(hi * 8, int(seq[b])))
    if len(toks):
        ref_s = brute.attention_over_tokens(list(q[b, h]), k[b, 0], v[b, 0], toks, scale)
        assert np.max(np.abs(o[b, h, s] - np.array(ref_s))) < 1e-12
    else:
        assert l[b, h, s] == 0 and m[b, h, s] == -math.inf


def test_block_range_and_two_level_merge():
    q, k, v, seq = rand_inputs(12, B=1, Hq=2, Hkv=1, d=8, L=64, ragged=False)
    scale = 0.4
    # 8 shards x 2 inner splits, merged per shard then across shards
    m, l, o = decode_split_states(q, k, v, seq, scale, 16, block=4)
    inner = merge_state_arrays(m.reshape(1, 2, 8, 2), l.reshape(1, 2, 8, 2), o.reshape(1, 2, 8, 2, 8))
    O2, _, _ = merge_state_arrays(inner[1], inner[2], inner[0])
    ref = decode_dense(q, k, v, seq, scale, block=4)
    assert np.max(np.abs(O2 - ref)) < 1e-12
    # a block range [3, 9) only
    m, l, o = decode_split_states(q, k, v, seq, scale, 2, block_begin=3, block_end=9, block=4)
    O, _, _ = merge_state_arrays(m, l, o)
    ref = brute.attention_over_tokens(list(q[0, 1]), k[0, 0], v[0, 0], range(12, 36), scale)
    assert np.max(np.abs(O[0, 1] - np.array(ref))) < 1e-12


def test_block_permutation_invariance():
    # ART summary §2.4: reordering KV blocks does not change softmax attention.
    q, k, v, seq = rand_inputs(13, B=1, Hq=2, Hkv=1, d=8, L=48, ragged=False)
    perm = np.random.default_rng(1).permutation(6)
    kp = k.reshape(1, 1, 6, 8, 8)[:, :, perm].reshape(k.shape)
    vp = v.reshape(1, 1, 6, 8, 8)[:, :, perm].reshape(v.shape)
    a = decode_dense(q, k, v, seq, 0.3, block=8)
    b = decode_dense(q, kp, vp, seq, 0.3, block=8)
    assert np.max(np.abs(a - b)) < 1e-13


def test_selected_blocks_attention():
    q, k, v, seq = rand_inputs(14, B=2, Hq=4, Hkv=2, d=8, L=40)
    lists = [[[0, 2, 4], [1, 4]], [[0, 3], [2]]]
    out = oracle.decode_blocks(q, k, v, seq, 0.3, lists, block=8)
    for b in range(2):
        for h in range(4):
            g = h // 2
            toks = [t for j in lists[b][g] for t in range(j * 8, min(j * 8 + 8, int(seq[b])))]
            ref = brute.attention_over_tokens(list(q[b, h]), k[b, g], v[b, g], toks, 0.3)
            assert np.max(np.abs(out[b, h] - np.array(ref))) < 1e-12
    # all blocks selected == dense
    nbs = [-(-int(s) // 8) for s in seq]
    full = [[list(range(nbs[b]))] * 2 for b in range(2)]
    assert np.max(np.abs(oracle.decode_blocks(q, k, v, seq, 0.3, full, block=8)
                         - decode_dense(q, k, v, seq, 0.3, block=8))) < 1e-13
    # split states over the selected list merge back to the same output
    m, l, o = oracle.decode_sparse_split_states(q, k, v, seq, 0.3, lists, 2, block=8)
    O, _, _ = merge_state_arrays(m, l, o)
    assert np.max(np.abs(O - out)) < 1e-12


def test_split_ranges_partition():
    for n in range(0, 20):
        for S in range(1, 9):
            rs = oracle.split_ranges(n, S)
            assert rs[0][0] == 0 and rs[-1][1] == n
            assert all(rs[i][1] == rs[i + 1][0] for i in range(S - 1))
            sizes = [hi - lo for lo, hi in rs]
            assert max(sizes) - min(sizes) <= 1
