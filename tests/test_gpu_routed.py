"""GPU parity: per-layer hard routing (full vs sink+window attention)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL, assert_close, log, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mask,n_shards,sps,sa_splits", [
    ([1, 0, 0, 1, 1, 0], 8, 2, 3),    # mixed stack
    ([1, 1, 1], 1, 1, 1),              # every layer full, one shard of one split
    ([0, 0, 0], 3, 5, 7),              # every layer sink + window
    ([0, 1, 1, 0], 8, 4, 32),          # the benchmark's split counts
    ([1, 0, 1], 9, 8, 5),              # 72 states per row: the two merge levels as separate launches
])
def test_routed_stack_matches_oracle(mask, n_shards, sps, sa_splits):
    log(f"[routed] {len(mask)}-layer stack {mask}, {n_shards} shards x {sps} splits, {sa_splits} SA splits; "
        "sink + window layers poisoned outside their blocks")
    n_layers, B, Hq, Hkv, d, L = len(mask), 2, 8, 2, 128, 64 * 40
    seq = [64 * 40, 64 * 29 + 3]
    n_sink, n_recent = 1, 6
    import sparse_kv_amd as skv

    layers, host = [], []
    lists = []
    for b in range(B):
        nb = -(-seq[b] // 64)
        f = sorted(oracle.selection.forced_blocks(nb, n_sink, n_recent))
        lists.append([f] * Hkv)
    for i in range(n_layers):
        inp = synth.make_inputs(50, B, Hq, Hkv, d, L, kind="needles", seq_lens=seq, layer=i)
        host.append(inp.f64())
        if not mask[i]:
            synth.poison_blocks(inp, lists)
        layers.append(upload(inp))
    sl = layers[0][3]
    idx, n = skv.attn_select_topk(None, sl, k=0, n_sink_blocks=n_sink, n_recent_blocks=n_recent,
                                  shape=(B, Hkv, L // 64))
    outs = skv.attn_decode_routed([x[0] for x in layers], [x[1] for x in layers], [x[2] for x in layers], mask,
                                  sl, n_shards=n_shards, splits_per_shard=sps, sa_block_idx=idx, sa_n_sel=n,
                                  sa_splits=sa_splits)
    torch.cuda.synchronize()
    ref = oracle.routed_layer_outputs(host, np.array(seq), 1 / np.sqrt(d), mask, n_sink, n_recent)
    for i in range(n_layers):
        assert_close(outs[i].cpu().numpy(), ref[i], TOL, f"layer {i} ({'FA' if mask[i] else 'SA'})")


def test_shard_aligned_two_level_merge_equals_one_level():
    log("[routed] shard-aligned splits merged twice == merged once")
    inp = synth.make_inputs(51, 1, 8, 2, 128, 64 * 37, kind="needles")
    q, k, v, sl = upload(inp)
    import sparse_kv_amd as skv

    m, l, o = skv.attn_decode_dense(q, k, v, sl, num_splits=8 * 3)
    so, sm, sl_ = skv.attn_merge_states(m.view(1, 8, 8, 3), l.view(1, 8, 8, 3), o.view(1, 8, 8, 3, 128),
                                        m_out=True, l_out=True)
    two = skv.attn_merge_states(sm, sl_, so)
    one = skv.attn_merge_states(m, l, o)
    torch.cuda.synchronize()
    assert_close(two.cpu().numpy(), one.cpu().numpy(), 2e-6, "two-level vs one-level")
    qf, kf, vf = inp.f64()
    assert_close(two.cpu().numpy(), oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale), TOL, "vs oracle")
