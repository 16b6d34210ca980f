"""Pins of the paged-cache gather (CPU only)."""

import numpy as np

from oracle.paged import gather_paged


def test_identity_table_gives_the_cache():
    r = np.random.default_rng(0)
    B, Hkv, nb, blk, d = 2, 3, 5, 4, 6
    cache = r.standard_normal((B, Hkv, nb * blk, d))
    pool = cache.reshape(B, Hkv, nb, blk, d).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, blk, d)
    table = np.arange(B * nb).reshape(B, nb)
    seq = np.array([nb * blk, 7])
    got = gather_paged(pool, table, seq, nb, block=blk)
    assert np.array_equal(got[0], cache[0])
    assert np.array_equal(got[1, :, :7], cache[1, :, :7]) and not got[1, :, 7:].any()


def test_permuted_pool_and_shared_blocks():
    r = np.random.default_rng(1)
    Hkv, blk, d = 2, 4, 3
    blocks = r.standard_normal((6, Hkv, blk, d))
    perm = r.permutation(6)
    pool = np.zeros((8, Hkv, blk, d))
    pool[perm] = blocks  # logical block i lives in slot perm[i]; slots 6, 7 unused
    pool[6:] = np.nan
    table = np.array([[perm[0], perm[1], perm[2]], [perm[0], perm[1], perm[5]]])  # rows share two blocks
    seq = np.array([12, 10])
    got = gather_paged(pool, table, seq, 3, block=blk)
    for j in range(3):
        assert np.array_equal(got[0, :, j * blk:(j + 1) * blk], blocks[j])
    assert np.array_equal(got[1, :, :8], got[0, :, :8])
    assert np.array_equal(got[1, :, 8:10], blocks[5][:, :2]) and not got[1, :, 10:].any()
    assert np.isfinite(got).all()
