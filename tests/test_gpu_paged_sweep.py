"""GPU parity: paged caches over a seeded sweep.

Each case scatters the logical blocks of seeded inputs over a permuted pool
(NaN in every unused slot and behind every table entry past a row's end,
optionally a shared prefix between two rows) and runs dense and listed-block
decode and both ART launch forms through the block table.  The split states
must be bit-identical to the contiguous cache's, the outputs within the
output tolerance of the oracle, and the ART stop positions exact.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL, assert_close, log, upload
from tests.test_gpu_paged import make_pool, up_pool

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(6000 + seed)
    B, Hkv = int(r.integers(2, 4)), int(r.integers(1, 3))
    G = int(r.choice([1, 2, 4, 5, 8]))
    d = int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    NB = int(r.integers(4, 33))
    L = 64 * NB
    seq = [int(x) for x in r.integers(0, L + 1, B)]
    seq[0] = L
    share = int(r.integers(0, min(4, -(-seq[1] // 64)) + 1))
    S = int(r.choice([1, 3, 7]))
    return B, Hkv, G, d, dt, L, seq, share, S


@pytest.mark.parametrize("seed", range(10))
def test_paged_decode_sweep(seed):
    import sparse_kv_amd as skv

    B, Hkv, G, d, dt, L, seq, share, S = _case(seed)
    log(f"[paged-sweep] seed={seed} B={B} Hq={Hkv * G} Hkv={Hkv} d={d} {dt} L={L} seq={seq} share={share} S={S}")
    inp = synth.make_inputs(110 + seed, B, Hkv * G, Hkv, d, L, dtype=dt, kind="needles", seq_lens=seq)
    kp, vp, table = make_pool(inp, 20 + seed, share_blocks=share)
    q, k, v, sl = upload(inp)
    kpd, vpd, tab = up_pool(kp, vp, table, dt)
    qf, kf, vf = inp.f64()

    st_p = skv.attn_decode_dense_paged(q, kpd, vpd, tab, sl, num_splits=S)
    st_c = skv.attn_decode_dense(q, k, v, sl, num_splits=S)
    out = skv.attn_merge_states(*st_p)
    torch.cuda.synchronize()
    for a, b in zip(st_p, st_c):
        assert torch.equal(a, b), "paged dense states differ from the contiguous cache's"
    assert_close(out.cpu().numpy(), oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale), TOL, "paged dense")

    r = np.random.default_rng(8000 + seed)
    width = L // 64
    lists, bi, ns = [], np.full((B, Hkv, width), -1, dtype=np.int32), np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        nb = -(-seq[b] // 64)
        row = []
        for g in range(Hkv):
            sel = oracle.select_blocks(r.standard_normal(width), nb, int(r.integers(0, width + 1)), 1, 2)
            row.append(sel)
            bi[b, g, :len(sel)] = sel
            ns[b, g] = len(sel)
        lists.append(row)
    bi_d, ns_d = torch.from_numpy(bi).cuda(), torch.from_numpy(ns).cuda()
    st_p = skv.attn_decode_sparse_paged(q, kpd, vpd, tab, bi_d, ns_d, sl, num_splits=S)
    st_c = skv.attn_decode_sparse(q, k, v, bi_d, ns_d, sl, num_splits=S)
    out = skv.attn_merge_states(*st_p)
    torch.cuda.synchronize()
    for a, b in zip(st_p, st_c):
        assert torch.equal(a, b), "paged listed-block states differ from the contiguous cache's"
    assert_close(out.cpu().numpy(), oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, lists), TOL,
                 "paged listed blocks")


@pytest.mark.parametrize("path", ["one", "ws"])
@pytest.mark.parametrize("seed", range(4))
def test_paged_art_sweep(seed, path):
    import sparse_kv_amd as skv
    from tests.test_gpu_art import P, PHI, PROBE, TAU, art_inputs

    B, Hkv, G, d, dt, L, seq, share, _ = _case(20 + seed)
    seq = [max(s, 64) for s in seq]
    log(f"[paged-sweep] ART seed={seed} ({path}) B={B} Hq={Hkv * G} Hkv={Hkv} d={d} {dt} L={L} seq={seq}")
    inp, ref_out, ref_stop = art_inputs(120 + seed, B, Hkv * G, Hkv, d, L, seq=seq, dtype=dt)
    kp, vp, table = make_pool(inp, 30 + seed)
    q, _, _, sl = upload(inp)
    kpd, vpd, tab = up_pool(kp, vp, table, dt)
    fn = skv.attn_decode_art_paged_ws if path == "ws" else skv.attn_decode_art_paged
    out, stop, _ = fn(q, kpd, vpd, tab, sl, tau=TAU, phi=PHI, patience=P, probe_dim=PROBE)
    torch.cuda.synchronize()
    assert np.array_equal(stop.cpu().numpy(), ref_stop)
    assert_close(out.cpu().numpy(), ref_out, TOL, "paged ART output")
