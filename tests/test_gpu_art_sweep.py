"""GPU parity: ART over a seeded sweep of shapes, thresholds and visit orders.

Each case draws batch, KV heads, group size (1..8, padded groups included),
head dimension, dtype, ragged sequence lengths, thresholds (tau, phi),
patience, probe width and either the default order or a per-row custom order
(block 0 first, the rest permuted); inputs are redrawn until every decision
clears the 1% band around the thresholds, so the stop positions are fixed.
Both launch forms must reproduce the oracle's stop positions exactly and its
outputs within the output tolerance, and fetch no fewer blocks than needed
nor more than their read-ahead allows.
"""

import numpy as np
import pytest

from tests.gpu_util import TOL, assert_close, log
from tests.test_gpu_art import PATHS, art_inputs, check_fetched, run_art

pytestmark = pytest.mark.gpu

THRESHOLDS = [(1e-3, 1e-4), (5e-3, 5e-4), (2e-2, 2e-3)]


def _case(seed):
    r = np.random.default_rng(7000 + seed)
    B, Hkv = int(r.integers(1, 4)), int(r.integers(1, 3))
    G = int(r.choice([1, 2, 3, 4, 5, 8]))
    d = int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    NB = int(r.integers(6, 41))
    L = 64 * NB
    seq = [int(x) for x in r.integers(64, L + 1, B)]
    seq[0] = L
    tau, phi = THRESHOLDS[seed % len(THRESHOLDS)]
    p = int(r.integers(1, 5))
    probe = int(r.choice([1, 3, 8, 12, 16]))
    recent = 64 * int(r.integers(2, max(3, NB // 2)))
    order = None
    if seed % 2 == 1:
        order = np.zeros((B, Hkv, NB), dtype=np.int32)
        for b in range(B):
            nb = -(-seq[b] // 64)
            for g in range(Hkv):
                order[b, g] = [0] + list(r.permutation(np.arange(1, nb))) + list(range(nb, NB))
    return B, Hkv, G, d, dt, L, seq, tau, phi, p, probe, recent, order


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("seed", range(12))
def test_art_sweep_matches_oracle(seed, path):
    B, Hkv, G, d, dt, L, seq, tau, phi, p, probe, recent, order = _case(seed)
    log(f"[art-sweep] seed={seed} ({path}) B={B} Hq={Hkv * G} Hkv={Hkv} d={d} {dt} L={L} seq={seq} "
        f"tau={tau} phi={phi} p={p} probe={probe} order={'custom' if order is not None else 'default'}")
    inp, ref_out, ref_stop = art_inputs(80 + seed, B, Hkv * G, Hkv, d, L, seq=seq, dtype=dt, recent=recent,
                                        order=order, tau=tau, phi=phi, p=p, probe=probe)
    out, stop, fetched = run_art(inp, order=order, tau=tau, phi=phi, p=p, probe=probe, path=path)
    assert np.array_equal(stop, ref_stop), (stop.tolist(), ref_stop.tolist())
    assert_close(out, ref_out, TOL, "ART output")
    check_fetched(fetched, stop, inp, path)
