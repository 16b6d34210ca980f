"""Centroid-based block selection (fp64 reference).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:

* Centroid: one representative per group of keys, the mean of the group --
  Squeezed Attention blog, Q1 (cluster centroids stored in place of the keys)
  and Q2 step 1.  Reading used here: the group is a block of 64 consecutive
  tokens, so c_j is the mean of block j's (valid) keys.
* Score: the query is compared with every centroid to decide which keys to
  load -- Squeezed Attention blog, Q1 and Q2 step 2.  Reading: the comparison
  is the scaled dot product (the mean logit of the block, by linearity).
  One score per GQA group, no softmax -- SparDA summary §2 (compact Forecast
  indexer); reading: the group's query vectors are summed,
  sigma_j = scale * <sum_{h in g} q_h, c_j>.
* Choice: the highest-scoring blocks are kept (top-k), and the first block
  (attention sink, ART summary §2.4; 64-token sink prefix, Pulsar Phase 1)
  plus a recent window are always kept.  Forced blocks do not compete for the
  k slots; ties go to the lower block index; the list is ascending.

Decision precision: the oracle computes scores in float64 and takes the
top-k comparison on the scores rounded to float32, the precision the
kernels decide in.  On inputs whose k-th / (k+1)-th gap exceeds 1e-4 the two
are the same decision.

* Two levels (Squeezed Attention blog, Q2 step 4, optional hierarchical
  clustering; Q1 on hierarchical clustering): coarse groups are searched
  first, then the fine groups inside the relevant coarse ones.  Reading: a
  coarse group is `group` consecutive blocks (a super-block) whose centroid
  is the mean of its valid keys; the coarse score is the same scaled dot
  product; the k_coarse best super-blocks that hold at least one non-forced
  block are kept (ties to the lower index), and the k fine picks are made
  among the non-forced blocks inside them.  Forced blocks are added as in the
  one-level choice.

Pins: tests/test_oracle_selection.py (the centroid/score identity against a
per-token pure-Python brute force, a brute-force sort, k >= |candidates|
selecting everything, constructed ties, and the Squeezed Attention worked
example of six keys in two clusters, tests/golden/squeezed_toy.json; for
two levels: super-block centroids against a per-token brute-force mean,
k_coarse covering every super-block and group = 1 both reducing to the
one-level choice, and a constructed case where the coarse level hides a
block the one-level choice would take).
The split of k versus forced blocks is a reading: parity unpinned beyond the
brute-force sort.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import num_blocks


def block_centroids(k, seq_lens, block: int = 64):
    """Mean key of every block: C [B, Hkv, NBmax, d] float64.

    NBmax = ceil(Lmax / block).  Blocks at or beyond nb(b) are zero; a
    partial last block averages its valid tokens only.
    """
    B, Hkv, Lmax, d = k.shape
    NBmax = num_blocks(Lmax, block)
    C = np.zeros((B, Hkv, NBmax, d))
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(num_blocks(L, block)):
            lo, hi = j * block, min((j + 1) * block, L)
            C[b, :, j] = k[b, :, lo:hi].mean(axis=1)
    return C


def centroid_scores(q, C, seq_lens, scale: float, block: int = 64):
    """Group scores sigma [B, Hkv, NBmax]; -inf at or beyond nb(b)."""
    B, Hq, d = q.shape
    Hkv = C.shape[1]
    G = Hq // Hkv
    NBmax = C.shape[2]
    sig = np.full((B, Hkv, NBmax), -math.inf)
    for b in range(B):
        nb = num_blocks(int(seq_lens[b]), block)
        for g in range(Hkv):
            qsum = q[b, g * G:(g + 1) * G].sum(axis=0)
            sig[b, g, :nb] = scale * (C[b, g, :nb] @ qsum)
    return sig


def forced_blocks(nb: int, n_sink: int, n_recent: int):
    """Sink blocks [0, n_sink) and the recent window [nb - n_recent, nb), clipped."""
    f = set(range(0, min(n_sink, nb)))
    f |= set(range(max(nb - n_recent, 0), nb))
    return f


def select_blocks(scores_row, nb: int, k: int, n_sink: int, n_recent: int):
    """Selected block indices (ascending) for one KV head.

    scores_row: the head's scores (only the first nb are read).  The forced
    set F is added on top of the min(k, |candidates|) best candidates, ranked
    by descending float32 score with the lower index first among equals.
    """
    F = forced_blocks(nb, n_sink, n_recent)
    cand = np.array([j for j in range(nb) if j not in F], dtype=np.int64)
    picks = []
    if k > 0 and cand.size:
        s32 = np.asarray(scores_row, dtype=np.float64)[cand].astype(np.float32)
        order = np.lexsort((cand, -s32.astype(np.float64)))
        picks = cand[order[:min(k, cand.size)]].tolist()
    return sorted(F | set(picks))


def select_all(scores, seq_lens, k: int, n_sink: int, n_recent: int, block: int = 64):
    """select_blocks for every (b, g): nested lists [B][Hkv]."""
    B, Hkv, _ = scores.shape
    out = []
    for b in range(B):
        nb = num_blocks(int(seq_lens[b]), block)
        out.append([select_blocks(scores[b, g], nb, k, n_sink, n_recent) for g in range(Hkv)])
    return out


def selection_gap(scores_row, nb: int, k: int, n_sink: int, n_recent: int):
    """Score gap between the k-th and (k+1)-th candidate (inf if no boundary).

    Used by the tests to certify that an input's selection is decided with a
    margin well above float32 rounding.
    """
    F = forced_blocks(nb, n_sink, n_recent)
    cand = [j for j in range(nb) if j not in F]
    if k <= 0 or k >= len(cand):
        return math.inf
    s = np.sort(np.asarray(scores_row, dtype=np.float64)[cand])[::-1]
    return float(s[k - 1] - s[k])


def super_centroids(k, seq_lens, group: int, block: int = 64):
    """Mean key of every super-block of `group` consecutive blocks:
    C2 [B, Hkv, ceil(NBmax / group), d]; zeros past the sequence's end."""
    B, Hkv, Lmax, d = k.shape
    span = group * block
    NS = -(-num_blocks(Lmax, block) // group)
    C = np.zeros((B, Hkv, NS, d))
    for b in range(B):
        L = int(seq_lens[b])
        for s_ in range(-(-L // span)):
            lo, hi = s_ * span, min((s_ + 1) * span, L)
            C[b, :, s_] = k[b, :, lo:hi].mean(axis=1)
    return C


def select_blocks_two_level(fine_row, coarse_row, nb: int, group: int, k_coarse: int, k: int,
                            n_sink: int, n_recent: int):
    """Two-level selection for one KV head (ascending block list).

    The super-blocks holding a non-forced block compete on their float32
    coarse score (lower index first among equals); the k_coarse best are
    opened and min(k, |their non-forced blocks|) blocks are picked among
    those on the float32 fine score (lower index first); forced blocks are
    added.
    """
    F = forced_blocks(nb, n_sink, n_recent)
    ns = -(-nb // group)
    members = {s_: [j for j in range(s_ * group, min((s_ + 1) * group, nb)) if j not in F] for s_ in range(ns)}
    eligible = [s_ for s_ in range(ns) if members[s_]]
    c32 = np.asarray(coarse_row, dtype=np.float64).astype(np.float32)
    opened = sorted(eligible, key=lambda s_: (-float(c32[s_]), s_))[:max(k_coarse, 0)]
    cand = sorted(j for s_ in opened for j in members[s_])
    f32 = np.asarray(fine_row, dtype=np.float64).astype(np.float32)
    picks = sorted(cand, key=lambda j: (-float(f32[j]), j))[:max(k, 0)]
    return sorted(F | set(picks))


def select_all_two_level(fine, coarse, seq_lens, group: int, k_coarse: int, k: int, n_sink: int,
                         n_recent: int, block: int = 64):
    """select_blocks_two_level for every (b, g): nested lists [B][Hkv]."""
    B, Hkv, _ = fine.shape
    out = []
    for b in range(B):
        nb = num_blocks(int(seq_lens[b]), block)
        out.append([select_blocks_two_level(fine[b, g], coarse[b, g], nb, group, k_coarse, k, n_sink, n_recent)
                    for g in range(Hkv)])
    return out


def two_level_gaps(fine_row, coarse_row, nb: int, group: int, k_coarse: int, k: int, n_sink: int,
                   n_recent: int):
    """(coarse gap, fine gap): the score gaps at the two decision boundaries
    (inf where there is no boundary), for certifying margins in tests."""
    F = forced_blocks(nb, n_sink, n_recent)
    ns = -(-nb // group)
    members = {s_: [j for j in range(s_ * group, min((s_ + 1) * group, nb)) if j not in F] for s_ in range(ns)}
    eligible = [s_ for s_ in range(ns) if members[s_]]
    cg = math.inf
    if 0 < k_coarse < len(eligible):
        cs = np.sort(np.asarray(coarse_row, dtype=np.float64)[eligible])[::-1]
        cg = float(cs[k_coarse - 1] - cs[k_coarse])
    c64 = np.asarray(coarse_row, dtype=np.float64)
    opened = sorted(eligible, key=lambda s_: (-c64[s_], s_))[:max(k_coarse, 0)]
    cand = [j for s_ in opened for j in members[s_]]
    fg = math.inf
    if 0 < k < len(cand):
        fs = np.sort(np.asarray(fine_row, dtype=np.float64)[cand])[::-1]
        fg = float(fs[k - 1] - fs[k])
    return cg, fg
