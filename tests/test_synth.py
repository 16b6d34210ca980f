"""Checks of the seeded input generators (CPU only)."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0, -2.5, 3.00390625, 1 + 2 ** -8, 1 + 3 * 2 ** -9], dtype=np.float32)])
    ours = synth.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_determinism_and_unit_redraw():
    a = synth.make_inputs(2, 2, 8, 2, 16, 256, kind="needles", threads=1)
    b = synth.make_inputs(2, 2, 8, 2, 16, 256, kind="needles", threads=4)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    c = synth.make_inputs(2, 2, 8, 2, 16, 256, kind="needles", attempts={(1, 0): 1})
    assert np.array_equal(a.k[0], c.k[0]) and np.array_equal(a.k[1, 1], c.k[1, 1])
    assert not np.array_equal(a.k[1, 0], c.k[1, 0]) and not np.array_equal(a.q[1, :4], c.q[1, :4])


def test_ragged_padding_is_nan_and_needles_avoid_block0():
    seq = np.array([100, 256])
    x = synth.make_inputs(2, 2, 4, 1, 8, 256, kind="needles", seq_lens=seq)
    kf = synth.bf16_to_f32(x.k)
    assert np.isnan(kf[0, 0, 100:]).all() and np.isfinite(kf[0, 0, :100]).all()
    assert np.isfinite(kf[1]).all()
    # needle keys have a large component along the group's summed query
    u = synth.bf16_to_f32(x.q[1]).astype(np.float64).sum(0)
    u /= np.linalg.norm(u)
    proj = kf[1, 0].astype(np.float64) @ u
    assert (proj[:64] < 3.5).all() and (proj > 2.0).sum() >= 12


def test_mixture_is_block_coherent():
    x = synth.make_inputs(3, 1, 4, 1, 16, 64 * 6, kind="mixture", dtype="f32")
    kb = x.k[0, 0].reshape(6, 64, 16)
    within = kb.std(axis=1).mean()
    assert 0.25 < within < 0.35


def test_route_mask():
    m = synth.route_mask(36, 18)
    assert m.sum() == 18 and m.dtype == np.uint8
    assert np.array_equal(m, synth.route_mask(36, 18))
