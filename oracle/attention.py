"""Decode attention, split states and their exact merge (fp64 reference).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:

* Streaming tile-wise decode attention: the output is accumulated as KV blocks
  are visited, and the intermediate (running max, denominator, output) state
  is exposed cheaply -- ART summary page, §2.1.  Here the state over a token
  set J is written out directly (no streaming): m = max_j s_j,
  l = sum_j exp(s_j - m), O = sum_j exp(s_j - m) v_j / l, with
  s_j = scale * <q, k_j>.  The empty set has the state (-inf, 0, 0).
* Exact merge of partial states by online softmax -- Pulsar summary page,
  Phase 2 (queries broadcast to every shard, local attention per shard,
  results combined by the online-softmax merge of Milakov and Gimelshein):
  M = max_r m_r, w_r = l_r exp(m_r - M), O = sum_r w_r O_r / sum_r w_r.
* Attention restricted to selected keys only -- Squeezed Attention blog, Q2
  step 3 ("Sparse FlashAttention" over the keys of the chosen clusters).

Layouts (all float64 numpy arrays): q [B, Hq, d]; k, v [B, Hkv, Lmax, d];
seq_lens int [B].  Query head h reads KV head h // G with G = Hq / Hkv
(grouped-query attention).  Blocks are ``block`` consecutive tokens; block j
of sequence b covers tokens [j*block, min((j+1)*block, L_b)).

Pins: tests/test_oracle_attention.py (pure-Python brute force on tiny inputs,
torch.softmax in float64 as an independent library routine, single-token and
identical-key closed forms, split+merge = unsplit on random partitions,
associativity, empty-state identities, invariance under block permutation).
"""

from __future__ import annotations

import math

import numpy as np

EMPTY_STATE = (-math.inf, 0.0, None)


def num_blocks(L: int, block: int = 64) -> int:
    """Number of blocks holding L tokens (the last one may be partial)."""
    return -(-int(L) // block)


def block_ranges(L: int, block: int = 64):
    """Token ranges [(lo, hi)] of the blocks of a length-L sequence."""
    return [(j * block, min((j + 1) * block, L)) for j in range(num_blocks(L, block))]


def split_ranges(n: int, num_splits: int):
    """Partition of n consecutive items into num_splits contiguous parts.

    Part s holds items [floor(s*n/S), floor((s+1)*n/S)).  Parts may be empty
    when n < S.  This partition is part of the library's interface (it fixes
    which split a block lands in), so the oracle states it explicitly.
    """
    S = int(num_splits)
    return [((s * n) // S, ((s + 1) * n) // S) for s in range(S)]


def head_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax state of one query over the token set given by the rows of K, V.

    Returns (m, l, O) with O normalised; (-inf, 0, zeros) for an empty set.
    """
    d = q.shape[-1]
    if K.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(d)
    s = scale * (K @ q)
    m = float(s.max())
    w = np.exp(s - m)
    l = float(w.sum())
    O = (w @ V) / l
    return m, l, O


def merge_states(states, d: int | None = None):
    """Exact online-softmax merge of partial states [(m, l, O), ...].

    Empty states (l == 0) are skipped.  If every state is empty the result is
    (-inf, 0, zeros(d)).  Returns (M, L, O) with L = sum_r l_r exp(m_r - M).
    """
    states = list(states)
    if d is None:
        for st in states:
            if st[2] is not None:
                d = len(st[2])
                break
    live = [st for st in states if st[1] > 0.0]
    if not live:
        return -math.inf, 0.0, np.zeros(d if d is not None else 0)
    M = max(st[0] for st in live)
    w = np.array([st[1] * math.exp(st[0] - M) for st in live])
    O = sum(wr * st[2] for wr, st in zip(w, live)) / w.sum()
    return M, float(w.sum()), O


def _tokens_of_blocks(blocks, L: int, block: int):
    idx = []
    for j in blocks:
        lo, hi = j * block, min((j + 1) * block, L)
        idx.extend(range(lo, hi))
    return np.asarray(idx, dtype=np.int64)


def decode_dense(q, k, v, seq_lens, scale: float, block: int = 64):
    """Full decode attention over the first L_b tokens of each sequence.

    Returns O [B, Hq, d] float64 (zeros for an empty sequence).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            g = h // G
            _, _, O = head_state(q[b, h], k[b, g, :L], v[b, g, :L], scale)
            out[b, h] = O
    return out


def decode_split_states(q, k, v, seq_lens, scale: float, num_splits: int,
                        block_begin: int = 0, block_end: int = -1, block: int = 64):
    """Per-split softmax states of decode attention over a block range.

    The block range of sequence b is [min(block_begin, e), e) with
    e = nb(b) if block_end < 0 else min(block_end, nb(b)); it is cut into
    num_splits contiguous parts by ``split_ranges``.  Returns
    m [B, Hq, S], l [B, Hq, S], o [B, Hq, S, d] (o normalised, zero when empty).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    S = int(num_splits)
    m = np.full((B, Hq, S), -math.inf)
    l = np.zeros((B, Hq, S))
    o = np.zeros((B, Hq, S, d))
    for b in range(B):
        L = int(seq_lens[b])
        nb = num_blocks(L, block)
        e = nb if block_end < 0 else min(block_end, nb)
        bb = min(block_begin, e)
        for s, (lo, hi) in enumerate(split_ranges(e - bb, S)):
            toks = _tokens_of_blocks(range(bb + lo, bb + hi), L, block)
            for h in range(Hq):
                g = h // G
                ms, ls, Os = head_state(q[b, h], k[b, g, toks], v[b, g, toks], scale)
                m[b, h, s], l[b, h, s], o[b, h, s] = ms, ls, Os
    return m, l, o


def decode_blocks(q, k, v, seq_lens, scale: float, block_lists, block: int = 64):
    """Attention restricted to the tokens of selected blocks (one list per KV head).

    block_lists[b][g] is an iterable of block indices for KV head g of
    sequence b; tokens at or beyond L_b are never included.  Returns
    O [B, Hq, d].
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            g = h // G
            toks = _tokens_of_blocks(sorted(block_lists[b][g]), L, block)
            _, _, O = head_state(q[b, h], k[b, g, toks], v[b, g, toks], scale)
            out[b, h] = O
    return out


def decode_sparse_split_states(q, k, v, seq_lens, scale: float, block_lists,
                               num_splits: int, block: int = 64):
    """Per-split states of selected-block attention.

    The selected list of KV head g (ascending) is cut into num_splits
    contiguous parts of list positions by ``split_ranges``.  Returns
    m, l [B, Hq, S] and o [B, Hq, S, d].
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    S = int(num_splits)
    m = np.full((B, Hq, S), -math.inf)
    l = np.zeros((B, Hq, S))
    o = np.zeros((B, Hq, S, d))
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(Hkv):
            lst = sorted(block_lists[b][g])
            for s, (lo, hi) in enumerate(split_ranges(len(lst), S)):
                toks = _tokens_of_blocks(lst[lo:hi], L, block)
                for h in range(g * G, (g + 1) * G):
                    ms, ls, Os = head_state(q[b, h], k[b, g, toks], v[b, g, toks], scale)
                    m[b, h, s], l[b, h, s], o[b, h, s] = ms, ls, Os
    return m, l, o


def merge_state_arrays(m, l, o):
    """Merge the last split axis of state arrays m, l [..., S], o [..., S, d].

    Returns (O [..., d], M [...], L [...]).
    """
    lead = m.shape[:-1]
    d = o.shape[-1]
    O = np.zeros(lead + (d,))
    M = np.full(lead, -math.inf)
    Ls = np.zeros(lead)
    for idx in np.ndindex(*lead):
        states = [(m[idx + (s,)], l[idx + (s,)], o[idx + (s,)]) for s in range(m.shape[-1])]
        M[idx], Ls[idx], O[idx] = merge_states(states, d)
    return O, M, Ls
