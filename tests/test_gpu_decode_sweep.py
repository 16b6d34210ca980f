"""GPU parity: dense and listed-block decode over a seeded sweep of shapes.

Each case draws batch, KV heads, group size (1..8, padded groups included),
head dimension, dtype, key distribution, ragged sequence lengths (empty,
one token, partial last block, full) and a split count that may exceed the
blocks; the listed-block case takes, per KV head, the ascending selection of
random scores with random k, sink and recent counts.  Split states and
merged outputs are compared with the oracle within the output tolerance,
and empty splits must be exactly (-inf, 0, 0).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL, assert_close, assert_states_close, log, upload

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(5000 + seed)
    B, Hkv = int(r.integers(1, 4)), int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 5, 6, 8]))
    d = int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    kind = str(r.choice(["gauss", "needles", "mixture"]))
    NB = int(r.integers(1, 41))
    L = 64 * NB
    seq = r.integers(0, L + 1, B)
    pick = r.integers(0, 4)
    seq[0] = [L, 0, 1, L - 17 if L > 17 else L][pick]
    S = int(r.choice([1, 2, 3, 5, 8, 13, 20]))
    return B, Hkv, G, d, dt, kind, L, [int(x) for x in seq], S


def _lists(r, seq, Hkv, L):
    B = len(seq)
    lists, n = [], np.zeros((B, Hkv), dtype=np.int32)
    width = L // 64
    idx = np.full((B, Hkv, max(width, 1)), -1, dtype=np.int32)
    for b in range(B):
        nb = -(-seq[b] // 64)
        row = []
        for g in range(Hkv):
            s = r.standard_normal(width)
            k, ns, nr = int(r.integers(0, width + 1)), int(r.integers(0, 3)), int(r.integers(0, 6))
            sel = oracle.select_blocks(s, nb, k, ns, nr)
            row.append(sel)
            n[b, g] = len(sel)
            idx[b, g, :len(sel)] = sel
        lists.append(row)
    return lists, idx, n


@pytest.mark.parametrize("seed", range(24))
def test_decode_sweep_matches_oracle(seed):
    import sparse_kv_amd as skv

    B, Hkv, G, d, dt, kind, L, seq, S = _case(seed)
    Hq = Hkv * G
    log(f"[decode-sweep] seed={seed} B={B} Hq={Hq} Hkv={Hkv} d={d} {dt} {kind} L={L} seq={seq} S={S}")
    inp = synth.make_inputs(70 + seed, B, Hq, Hkv, d, L, dtype=dt, kind=kind, seq_lens=seq)
    q, k, v, sl = upload(inp)
    qf, kf, vf = inp.f64()

    m, l, o = skv.attn_decode_dense(q, k, v, sl, num_splits=S)
    out = skv.attn_merge_states(m, l, o)
    torch.cuda.synchronize()
    rm, rl, ro = oracle.decode_split_states(qf, kf, vf, inp.seq_lens, inp.scale, S)
    assert_states_close(m, l, o, rm, rl, ro, TOL, "dense split states")
    assert_close(out.cpu().numpy(), oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale), TOL, "dense output")

    r = np.random.default_rng(9000 + seed)
    lists, idx, n = _lists(r, seq, Hkv, L)
    bi, ns_ = torch.from_numpy(idx).cuda(), torch.from_numpy(n).cuda()
    m, l, o = skv.attn_decode_sparse(q, k, v, bi, ns_, sl, num_splits=S)
    out = skv.attn_merge_states(m, l, o)
    torch.cuda.synchronize()
    rm, rl, ro = oracle.decode_sparse_split_states(qf, kf, vf, inp.seq_lens, inp.scale, lists, S)
    assert_states_close(m, l, o, rm, rl, ro, TOL, "listed split states")
    assert_close(out.cpu().numpy(), oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, lists), TOL,
                 "listed output")
