"""ART run-time termination of streaming decode attention (fp64 reference).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Steps followed, in the order of the ART technical summary (gist.science,
paper 2606.00024):

* §2.1: KV blocks are folded into the running attention state one at a time
  in a visit order; after t+1 blocks the partial output O^(t) is available.
* §2.4: the visit order may be re-arranged ("recency first" or "importance
  first"); the first block (block 0, the attention sink) is always evaluated
  before any early exit.  Default order here: (0, nb-1, nb-2, ..., 1);
  importance first: block 0, then descending centroid score.  ART composes
  with KV selection (§2.4, orthogonal control layer): the visit order may
  list only some blocks, and then attention is over those blocks.
* §2.2: a small probe vector x^(t) is read from the partial output.  Reading:
  x^(t) = the first ``probe_dim`` channels of the normalised partial output
  (the output if attention stopped now).  Two changes are measured against
  the previous probe: the magnitude change
  d_scale = | ||x^(t)|| - ||x^(t-1)|| |  (reading of "L2-norm difference"; the
  alternative ||x^(t) - x^(t-1)|| is not used -- parity unpinned for this
  choice) and the direction change d_dir = 1 - cos(x^(t), x^(t-1)), treated
  as not stable when either norm is zero.  A step is stable only if both
  fall strictly below their thresholds (tau, phi).
* §2.3: termination needs the criterion to hold for p consecutive blocks.
  The first comparison is at t = 1; the stop is the first t with a run of p
  stable steps ending at t; with no stop the whole sequence is folded.

Decision precision: d_scale and d_dir are computed in float64 and rounded to
float32 before the strict comparison with float32(tau), float32(phi) -- the
precision the kernel decides in.  Inputs whose every decision clears a 1%
band around the thresholds decide identically in both precisions.

Pins: tests/test_oracle_art.py (tau = phi = 0 and p > nb give dense
attention, tau = phi = inf with p = 1 stops at t = 1 with attention over the
first two visited blocks by brute force, the constant-probe construction
stops at exactly j + p, known-angle and known-norm probe pairs for the two
metrics, invariance of the dense result over any visit order that starts
with block 0, probe_dim = 0 disables the detector).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import head_state, merge_states, num_blocks


def default_order(nb: int):
    """Block 0 first, then the most recent block backwards: (0, nb-1, ..., 1)."""
    if nb <= 0:
        return []
    return [0] + list(range(nb - 1, 0, -1))


def importance_order(scores_row, nb: int):
    """Block 0 first, then the other blocks by descending score ("importance
    first", ART summary §2.4), lower index first among equal float32 scores."""
    if nb <= 0:
        return []
    s32 = np.asarray(scores_row, dtype=np.float64)[:nb].astype(np.float32)
    rest = sorted(range(1, nb), key=lambda j: (-float(s32[j]), j))
    return [0] + rest


def probe_metrics(x_cur, x_prev):
    """(d_scale, d_dir) between two probe vectors; d_dir = inf if a norm is 0."""
    n1 = math.sqrt(float(np.dot(x_cur, x_cur)))
    n0 = math.sqrt(float(np.dot(x_prev, x_prev)))
    d_scale = abs(n1 - n0)
    if n1 == 0.0 or n0 == 0.0:
        return d_scale, math.inf
    d_dir = 1.0 - float(np.dot(x_cur, x_prev)) / (n1 * n0)
    return d_scale, d_dir


def is_stable(d_scale, d_dir, tau, phi):
    """Strict 'both below' test, decided in float32."""
    return bool(np.float32(d_scale) < np.float32(tau) and np.float32(d_dir) < np.float32(phi))


def art_decode_head(q, K, V, L: int, scale: float, order, tau: float, phi: float,
                    patience: int, probe_dim: int, block: int = 64):
    """ART for one query head over one KV head.

    q [d]; K, V [Lmax, d] float64; ``order``: the visit order, distinct blocks
    of the sequence starting with 0 -- all nb of them, or fewer to visit only
    those (ART over a selected list).  Returns (O [d], T, trace) where T is the
    visit position of the last folded block (-1 when nothing is visited) and
    trace lists (t, d_scale, d_dir, stable, counter) for every compared step.
    """
    d = q.shape[-1]
    nb = num_blocks(L, block)
    order = list(order)[:nb]
    if not order:
        return np.zeros(d), -1, []
    state = (-math.inf, 0.0, np.zeros(d))
    x_prev = None
    counter = 0
    trace = []
    T = len(order) - 1
    for t, j in enumerate(order):
        lo, hi = j * block, min((j + 1) * block, L)
        state = merge_states([state, head_state(q, K[lo:hi], V[lo:hi], scale)], d)
        if probe_dim <= 0:
            continue
        x = state[2][:probe_dim]
        if t >= 1:
            ds, dd = probe_metrics(x, x_prev)
            st = is_stable(ds, dd, tau, phi)
            counter = counter + 1 if st else 0
            trace.append((t, ds, dd, st, counter))
            if counter >= patience:
                T = t
                break
        x_prev = x
    return state[2], T, trace


def art_decode(q, k, v, seq_lens, scale: float, tau: float, phi: float, patience: int,
               probe_dim: int, order=None, n_visit=None, block: int = 64):
    """ART for every (b, h).  order: None (default order) or int [B, Hkv, NBmax];
    n_visit: None (visit nb blocks) or int [B, Hkv] (visit only the first
    n_visit entries of the order).

    Returns (out [B, Hq, d], stop [B, Hq] int, traces dict (b, h) -> trace).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    stop = np.full((B, Hq), -1, dtype=np.int64)
    traces = {}
    for b in range(B):
        L = int(seq_lens[b])
        nb = num_blocks(L, block)
        for h in range(Hq):
            g = h // G
            ordr = default_order(nb) if order is None else [int(x) for x in order[b][g][:nb]]
            if n_visit is not None:
                ordr = ordr[:max(0, min(int(n_visit[b][g]), nb))]
            O, T, tr = art_decode_head(q[b, h], k[b, g], v[b, g], L, scale, ordr, tau, phi,
                                       patience, probe_dim, block)
            out[b, h], stop[b, h], traces[(b, h)] = O, T, tr
    return out, stop, traces


def art_margin_ok(trace, tau: float, phi: float, band: float = 0.01) -> bool:
    """True when every decision in the trace clears a relative band.

    Stable steps need d_scale < (1-band) tau and d_dir < (1-band) phi;
    unstable steps need d_scale > (1+band) tau or d_dir > (1+band) phi.
    """
    for _, ds, dd, st, _ in trace:
        if st:
            if not (ds < (1 - band) * tau and dd < (1 - band) * phi):
                return False
        else:
            if not (ds > (1 + band) * tau or dd > (1 + band) * phi):
                return False
    return True
