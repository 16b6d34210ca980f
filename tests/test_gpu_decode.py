"""GPU parity: split-KV dense decode and the state merge against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL, assert_close, assert_states_close, log, upload

pytestmark = pytest.mark.gpu

# (label, B, Hq, Hkv, d, Lmax, dtype, kind, seq_lens, num_splits)
CASES = [
    ("tiny-fp32-single-head-4K", 1, 1, 1, 64, 4096, "f32", "gauss", None, 4),
    ("bf16-g4-d128-ragged", 3, 8, 2, 128, 64 * 37, "bf16", "needles", [64 * 37, 1000, 65], 5),
    ("bf16-g8-d64", 2, 8, 1, 64, 64 * 20, "bf16", "gauss", [1280, 700], 3),
    ("f32-g2-d128", 2, 4, 2, 128, 64 * 10, "f32", "gauss", [640, 1], 2),
    ("bf16-g1-d128-more-splits-than-blocks", 1, 2, 2, 128, 64 * 9, "bf16", "gauss", None, 16),
    ("bf16-g4-empty-row", 2, 8, 2, 128, 64 * 6, "bf16", "gauss", [0, 300], 3),
    ("f32-g4-d64", 2, 8, 2, 64, 64 * 11, "f32", "needles", [64 * 11, 64 * 5 + 7], 4),
    ("bf16-g3-d128", 1, 6, 2, 128, 64 * 12, "bf16", "gauss", [64 * 12 - 5], 3),
    ("bf16-g6-d128-padded-heads", 2, 12, 2, 128, 64 * 13, "bf16", "needles", [64 * 13, 64 * 6 + 33], 4),
    ("f32-g8-d128", 1, 8, 1, 128, 64 * 7, "f32", "gauss", [64 * 7 - 1], 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dense_states_and_merge(case):
    label, B, Hq, Hkv, d, L, dt, kind, seq, S = case
    log(f"[dense] {label}")
    inp = synth.make_inputs(20, B, Hq, Hkv, d, L, dtype=dt, kind=kind, seq_lens=seq)
    q, k, v, sl = upload(inp)
    import sparse_kv_amd as skv

    m, l, o = skv.attn_decode_dense(q, k, v, sl, num_splits=S)
    out, mo, lo = skv.attn_merge_states(m, l, o, m_out=True, l_out=True)
    torch.cuda.synchronize()
    qf, kf, vf = inp.f64()
    rm, rl, ro = oracle.decode_split_states(qf, kf, vf, inp.seq_lens, inp.scale, S)
    assert_states_close(m, l, o, rm, rl, ro, TOL, "split states")
    ref = oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale)
    assert_close(out.cpu().numpy(), ref, TOL, "merged output")
    RO, RM, RL = oracle.attention.merge_state_arrays(rm, rl, ro)
    mo, lo = mo.cpu().numpy(), lo.cpu().numpy()
    live = RL > 0
    assert np.array_equal(lo > 0, live)
    assert np.all(np.isneginf(mo[~live]))
    if live.any():
        assert np.max(np.abs(mo[live] - RM[live])) < 1e-4 * max(1.0, np.abs(RM[live]).max())
        assert np.max(np.abs(lo[live] - RL[live]) / RL[live]) < 1e-4


def test_block_range_and_determinism():
    log("[dense] block range + run-to-run determinism")
    inp = synth.make_inputs(21, 2, 8, 2, 128, 64 * 30, kind="gauss", seq_lens=[64 * 30, 64 * 12 + 3])
    q, k, v, sl = upload(inp)
    import sparse_kv_amd as skv

    m, l, o = skv.attn_decode_dense(q, k, v, sl, num_splits=3, block_begin=4, block_end=20)
    m2, l2, o2 = skv.attn_decode_dense(q, k, v, sl, num_splits=3, block_begin=4, block_end=20)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(m, m2) and torch.equal(l, l2)
    qf, kf, vf = inp.f64()
    rm, rl, ro = oracle.decode_split_states(qf, kf, vf, inp.seq_lens, inp.scale, 3, block_begin=4, block_end=20)
    assert_states_close(m, l, o, rm, rl, ro, TOL, "range states")


@pytest.mark.parametrize("S", [1, 7, 16, 17, 64, 100])
def test_merge_random_states(S):
    # one split, the first output chunk (16 splits) and past it, one and two rounds of 64 states
    log(f"[merge] random states with empty entries, S={S}")
    r = np.random.default_rng(5 + S)
    rows, d = 37, 128
    m = r.standard_normal((rows, S)) * 4
    l = np.exp(r.standard_normal((rows, S)))
    o = r.standard_normal((rows, S, d))
    empty = r.random((rows, S)) < 0.3
    empty[3] = True  # a row with nothing at all
    m[empty], l[empty], o[empty] = -np.inf, 0.0, 0.0
    import sparse_kv_amd as skv

    t = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()
    out, mo, lo = skv.attn_merge_states(t(m), t(l), t(o), m_out=True, l_out=True)
    torch.cuda.synchronize()
    RO, RM, RL = oracle.attention.merge_state_arrays(m.astype(np.float32).astype(np.float64),
                                                     l.astype(np.float32).astype(np.float64),
                                                     o.astype(np.float32).astype(np.float64))
    assert_close(out.cpu().numpy(), RO, 1e-5, "merge output")
    assert np.isneginf(mo.cpu().numpy()[3]) and lo.cpu().numpy()[3] == 0 and not out[3].any()
    # an empty state's output is never used: NaN there changes nothing
    on = o.copy()
    on[empty] = np.nan
    outn = skv.attn_merge_states(t(m), t(l), t(on))
    torch.cuda.synchronize()
    assert torch.equal(outn, out), "NaN in an empty state's output reached the merge"
    for dd in (64,):
        o64 = o[..., :dd].copy()
        out64 = skv.attn_merge_states(t(m), t(l), t(o64))
        torch.cuda.synchronize()
        R64, _, _ = oracle.attention.merge_state_arrays(m.astype(np.float32).astype(np.float64),
                                                        l.astype(np.float32).astype(np.float64),
                                                        o64.astype(np.float32).astype(np.float64))
        assert_close(out64.cpu().numpy(), R64, 1e-5, "merge output d=64")


def test_nan_past_sequence_end_is_never_read():
    # synth pads every row past its length with NaN; outputs must stay finite
    log("[dense] NaN padding past the sequence end")
    inp = synth.make_inputs(22, 2, 4, 1, 128, 64 * 8, kind="gauss", seq_lens=[64 * 3 + 1, 64 * 8])
    assert np.isnan(synth.bf16_to_f32(inp.k[0, 0, 64 * 3 + 1:])).all()
    q, k, v, sl = upload(inp)
    import sparse_kv_amd as skv

    m, l, o = skv.attn_decode_dense(q, k, v, sl, num_splits=2)
    out = skv.attn_merge_states(m, l, o)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    qf, kf, vf = inp.f64()
    assert_close(out.cpu().numpy(), oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale), TOL, "output")
