"""Pins of the per-layer routing oracle (CPU only)."""

import numpy as np

import oracle


def layer(seed, L=40):
    r = np.random.default_rng(seed)
    return (r.standard_normal((1, 4, 8)), r.standard_normal((1, 2, L, 8)), r.standard_normal((1, 2, L, 8)))


def test_window_covering_sequence_equals_full_attention():
    layers = [layer(0), layer(1), layer(2)]
    seq = np.array([40])
    fa = oracle.routed_layer_outputs(layers, seq, 0.3, [1, 1, 1], 1, 2, block=8)
    sa_all = oracle.routed_layer_outputs(layers, seq, 0.3, [0, 0, 0], 1, 5, block=8)
    for a, b in zip(fa, sa_all):
        assert np.max(np.abs(a - b)) < 1e-13


def test_sink_window_layer_reads_only_its_blocks():
    q, k, v = layer(3)
    seq = np.array([40])
    ref = oracle.routed_layer_outputs([(q, k, v)], seq, 0.3, [0], 1, 2, block=8)[0]
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 8:24] = np.nan  # blocks 1 and 2 are outside the sink + window
    v2[:, :, 8:24] = np.nan
    out = oracle.routed_layer_outputs([(q, k2, v2)], seq, 0.3, [0], 1, 2, block=8)[0]
    assert np.isfinite(out).all() and np.max(np.abs(out - ref)) == 0
    lists = [[[0, 3, 4]] * 2]
    assert np.max(np.abs(out - oracle.decode_blocks(q, k, v, seq, 0.3, lists, block=8))) < 1e-15
