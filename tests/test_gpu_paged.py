"""GPU parity: paged KV cache (block pool + block table) for dense, listed-block
and ART decode and for centroids, against the oracle on the logical cache."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.art import art_margin_ok
from oracle.paged import gather_paged
from tests.gpu_util import TOL, assert_close, log, to_dev, upload

pytestmark = pytest.mark.gpu


def make_pool(inp, seed, extra=7, share_blocks=0):
    """Scatter the logical blocks of `inp` over a permuted pool.

    Unused pool slots hold NaN; table entries past a row's end point at a NaN
    slot.  With share_blocks = m, row 1's first m blocks are row 0's (inp's
    row 1 data is overwritten to match, so the oracle sees the same cache).
    Returns (k_pool, v_pool, table) as numpy arrays in inp's storage type.
    """
    B, _, Hkv, d, Lmax = inp.shape
    NB = Lmax // 64
    if share_blocks:
        n = 64 * share_blocks
        inp.k[1, :, :n] = inp.k[0, :, :n]
        inp.v[1, :, :n] = inp.v[0, :, :n]
    nbs = [-(-int(L) // 64) for L in inp.seq_lens]
    need = sum(nbs) - (min(share_blocks, nbs[1]) if share_blocks else 0)
    P = need + extra
    r = np.random.default_rng(seed)
    perm = r.permutation(P)
    nan = synth.BF16_NAN if inp.dtype == "bf16" else np.float32(np.nan)
    kp = np.full((P, Hkv, 64, d), nan, dtype=inp.k.dtype)
    vp = np.full((P, Hkv, 64, d), nan, dtype=inp.v.dtype)
    junk = int(perm[-1])  # never holds data
    table = np.full((B, NB), junk, dtype=np.int32)
    nxt = 0
    for b in range(B):
        for j in range(nbs[b]):
            if b == 1 and j < share_blocks:
                table[b, j] = table[0, j]
                continue
            slot = int(perm[nxt])
            nxt += 1
            kp[slot] = inp.k[b, :, 64 * j:64 * j + 64]
            vp[slot] = inp.v[b, :, 64 * j:64 * j + 64]
            table[b, j] = slot
    assert nxt == need and junk not in set(table[table != junk].ravel().tolist())
    return kp, vp, table


def up_pool(kp, vp, table, dtype):
    return to_dev(kp, dtype), to_dev(vp, dtype), torch.from_numpy(table).cuda()


def test_gather_matches_the_logical_cache():
    # the helper itself: gathering the pool reproduces the (finite part of the) logical cache
    inp = synth.make_inputs(70, 2, 4, 2, 64, 64 * 6, dtype="f32", kind="gauss", seq_lens=[64 * 6, 64 * 4 + 5])
    kp, vp, table = make_pool(inp, 1, share_blocks=2)
    kf = inp.upcast(inp.k)
    got = gather_paged(kp.astype(np.float64), table, inp.seq_lens, 6)
    for b in range(2):
        L = int(inp.seq_lens[b])
        assert np.array_equal(got[b, :, :L], kf[b, :, :L])


@pytest.mark.parametrize("label,dt,d,Hq,Hkv,seq,share", [
    ("bf16 d128 g4 shared prefix", "bf16", 128, 8, 2, [64 * 37, 64 * 29 + 17, 64 * 11], 5),
    ("f32 d64 g1", "f32", 64, 2, 2, [64 * 21, 1, 64 * 9 + 63], 0),
    ("bf16 d128 g8", "bf16", 128, 8, 1, [64 * 33, 64 * 33], 33),
])
def test_dense_and_listed_decode_paged(label, dt, d, Hq, Hkv, seq, share):
    import sparse_kv_amd as skv

    log(f"[paged] dense + listed-block decode: {label}")
    B = len(seq)
    Lmax = 64 * 37
    inp = synth.make_inputs(71, B, Hq, Hkv, d, Lmax, dtype=dt, kind="needles", seq_lens=seq)
    kp, vp, table = make_pool(inp, 2, share_blocks=share)
    q, k, v, sl = upload(inp)
    kpd, vpd, tab = up_pool(kp, vp, table, dt)
    S = 5
    m, l, o = skv.attn_decode_dense_paged(q, kpd, vpd, tab, sl, num_splits=S)
    out = skv.attn_merge_states(m, l, o)
    ref_gpu = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, sl, num_splits=S))
    # listed blocks: every third block plus the sink and the last block
    nb = [-(-s // 64) for s in seq]
    lists = [[sorted({0, max(n - 1, 0)} | set(range(0, n, 3))) if n else [] for _ in range(Hkv)] for n in nb]
    ms = max(len(x) for row in lists for x in row)
    bi = np.full((B, Hkv, ms), -1, dtype=np.int32)
    ns = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            bi[b, g, :len(lists[b][g])] = lists[b][g]
            ns[b, g] = len(lists[b][g])
    sp = skv.attn_merge_states(*skv.attn_decode_sparse_paged(q, kpd, vpd, tab, torch.from_numpy(bi).cuda(),
                                                             torch.from_numpy(ns).cuda(), sl, num_splits=3))
    torch.cuda.synchronize()
    qf, kf, vf = inp.f64()
    assert_close(out.cpu().numpy(), oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale), TOL, "paged dense")
    assert_close(out.cpu().numpy(), ref_gpu.cpu().numpy(), 1e-6, "paged vs contiguous dense")
    assert_close(sp.cpu().numpy(), oracle.decode_blocks(qf, kf, vf, inp.seq_lens, inp.scale, lists), TOL,
                 "paged listed blocks")


def test_centroids_paged():
    import sparse_kv_amd as skv

    log("[paged] centroid build and update")
    seq = np.array([64 * 20, 64 * 7 + 3, 64 * 12], dtype=np.int32)
    old = np.array([64 * 18 + 5, 64 * 7 + 1, 64 * 12], dtype=np.int32)
    inp = synth.make_inputs(72, 3, 4, 2, 128, 64 * 20, kind="mixture", seq_lens=seq)
    kp, vp, table = make_pool(inp, 3, share_blocks=4)
    q, k, v, sl = upload(inp)
    kpd, _, tab = up_pool(kp, vp, table, "bf16")
    C = skv.attn_build_centroids_paged(kpd, tab, torch.from_numpy(old).cuda())
    skv.attn_update_centroids_paged(kpd, tab, C, sl, prev_lens=torch.from_numpy(old).cuda(), span_hint=2)
    C_full = skv.attn_build_centroids_paged(kpd, tab, sl)
    torch.cuda.synchronize()
    _, kf, _ = inp.f64()
    ref = oracle.block_centroids(kf, inp.seq_lens)
    assert_close(C_full.cpu().numpy(), ref, 1e-5, "paged centroids")
    assert_close(C.cpu().numpy(), ref, 1e-5, "paged centroids built then updated")


@pytest.mark.parametrize("path", ["one", "ws"])
def test_art_paged(path):
    import sparse_kv_amd as skv
    from tests.test_gpu_art import P, PHI, PROBE, TAU, art_inputs

    log(f"[paged] ART stop positions, {path}")
    inp, ref_out, ref_stop = art_inputs(73, 2, 8, 2, 128, 64 * 40, seq=[64 * 40, 64 * 33 + 9])
    kp, vp, table = make_pool(inp, 4)
    q, k, v, sl = upload(inp)
    kpd, vpd, tab = up_pool(kp, vp, table, "bf16")
    fn = skv.attn_decode_art_paged_ws if path == "ws" else skv.attn_decode_art_paged
    out, stop, fetched = fn(q, kpd, vpd, tab, sl, tau=TAU, phi=PHI, patience=P, probe_dim=PROBE)
    torch.cuda.synchronize()
    assert np.array_equal(stop.cpu().numpy(), ref_stop)
    assert_close(out.cpu().numpy(), ref_out, TOL, "paged ART output")
