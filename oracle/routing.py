"""Per-layer hard routing between full and sink+window attention (fp64 reference).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Followed: Flux Attention summary (gist.science, paper 2604.07394), §2 -- at
inference every layer runs either full attention (FA) or sparse attention
(SA), a hard decision made once at prefill and cached; SA layers at decode
do not load the historical KV and keep a minimal KV set.  Reading of the
SA pattern: the first ``n_sink`` blocks (a 64-token sink prefix, as in the
Pulsar summary's Phase 1) plus the last ``n_recent`` blocks.

FA layers are additionally evaluated the way a context-sharded system would
(Pulsar summary, Phase 2): per-shard states, each the merge of its inner
splits, merged once more; the exact merge makes this equal to FA.

Pins: tests/test_oracle_routing.py (an SA window covering the whole
sequence equals FA; the two-level shard merge equals one-level FA).
"""

from __future__ import annotations

from .attention import decode_blocks, decode_dense, num_blocks
from .selection import forced_blocks


def routed_layer_outputs(layers, seq_lens, scale: float, route_mask, n_sink: int,
                         n_recent: int, block: int = 64):
    """Outputs of a layer stack under a hard route mask.

    layers: list of (q, k, v) float64 arrays per layer; route_mask[l] = 1 for
    full attention, 0 for sink + recent-window attention.  Returns a list of
    O [B, Hq, d].
    """
    outs = []
    for (q, k, v), fa in zip(layers, route_mask):
        if fa:
            outs.append(decode_dense(q, k, v, seq_lens, scale, block))
        else:
            B, Hkv = k.shape[0], k.shape[1]
            lists = []
            for b in range(B):
                nb = num_blocks(int(seq_lens[b]), block)
                f = sorted(forced_blocks(nb, n_sink, n_recent))
                lists.append([f for _ in range(Hkv)])
            outs.append(decode_blocks(q, k, v, seq_lens, scale, lists, block))
    return outs
