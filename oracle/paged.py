"""Paged KV cache: logical blocks mapped to a shared pool (fp64 reference).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reading (the pages name a block-organised cache -- ART summary §2.1, 64-token
tiles; SparDA summary, paged offload of blocks -- but fix no layout): a pool
holds physical blocks [P, Hkv, 64, d]; a block table [B, >= nb] maps logical
block j of row b to its physical block.  Attention over a paged cache is
attention over the logical cache this mapping gathers, so every other oracle
function applies unchanged to the result of gather_paged.

Pins: tests/test_oracle_paged.py (an identity table over a reshaped cache
gives the cache back, a permuted pool with the inverse permutation in the
table gives it back, rows sharing physical blocks see the same keys, and
positions past each row's length are zero).
"""

from __future__ import annotations

import numpy as np

from .attention import num_blocks


def gather_paged(pool, table, seq_lens, nb_max: int, block: int = 64):
    """Logical cache [B, Hkv, nb_max * block, d] from pool [P, Hkv, block, d]
    and table [B, >= nb(b)]: logical block j of row b is pool[table[b][j]];
    positions at or past each row's length are zero."""
    P, Hkv, blk, d = pool.shape
    assert blk == block
    B = len(seq_lens)
    out = np.zeros((B, Hkv, nb_max * block, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(num_blocks(L, block)):
            p = int(table[b][j])
            n = min(block, L - j * block)
            out[b, :, j * block:j * block + n] = pool[p, :, :n]
    return out
