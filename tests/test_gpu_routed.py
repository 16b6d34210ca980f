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


def _stack(seed, mask, B, Hq, Hkv, d, seq, n_sink, n_recent):
    """Device layers (sink + window layers poisoned outside their blocks) and their float64 copies."""
    L = 64 * max(1, -(-max(seq) // 64))
    lists = []
    for b in range(B):
        nb = -(-seq[b] // 64)
        lists.append([sorted(oracle.selection.forced_blocks(nb, n_sink, n_recent))] * Hkv)
    layers, host = [], []
    for i in range(len(mask)):
        inp = synth.make_inputs(seed, B, Hq, Hkv, d, L, kind="needles", seq_lens=seq, layer=i)
        host.append(inp.f64())
        if not mask[i]:
            synth.poison_blocks(inp, lists)
        layers.append(upload(inp))
    return layers, host, L


@pytest.mark.parametrize("G,d,seq", [
    (8, 64, [0, 64 * 21 + 5, 64 * 30]),   # G = 8, 1 channel per lane in the merges
    (4, 128, [1, 0, 64 * 9]),              # a one-token row, an empty row, splits with no blocks
])
def test_routed_shapes_and_reused_workspace(G, d, seq):
    """8 query heads per KV head (two rows per merge wave group), head dim 64, rows with no tokens or
    one token, splits with no blocks.  The workspace starts as 0xFF bytes and the same workspace
    serves two calls on different stacks: both match the oracle (no state is read before it is
    written)."""
    import sparse_kv_amd as skv

    B, Hkv = len(seq), 2
    Hq = G * Hkv
    mask, n_shards, sps, sa_splits, n_sink, n_recent = [1, 0, 1, 0], 4, 3, 6, 1, 4
    log(f"[routed] G {G}, d {d}, seq {seq}, {n_shards} shards x {sps} splits, {sa_splits} SA splits")
    ws = None
    for seed in (52, 53):
        layers, host, L = _stack(seed, mask, B, Hq, Hkv, d, seq, n_sink, n_recent)
        if ws is None:
            need = skv.attn_routed_workspace_bytes(layers[0][0], layers[0][1], n_shards, sps, sa_splits)
            ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        sl = layers[0][3]
        idx, n = skv.attn_select_topk(None, sl, k=0, n_sink_blocks=n_sink, n_recent_blocks=n_recent,
                                      shape=(B, Hkv, L // 64))
        outs = skv.attn_decode_routed([x[0] for x in layers], [x[1] for x in layers], [x[2] for x in layers],
                                      mask, sl, n_shards=n_shards, splits_per_shard=sps, sa_block_idx=idx,
                                      sa_n_sel=n, sa_splits=sa_splits, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.routed_layer_outputs(host, np.array(seq), 1 / np.sqrt(d), mask, n_sink, n_recent)
        for i in range(len(mask)):
            assert_close(outs[i].cpu().numpy(), ref[i], TOL, f"seed {seed} layer {i}")


def test_routed_stack_graph_replays():
    """The routed stack (a decode and its merges per layer) captured in a HIP graph: every replay,
    with new queries copied in and eager work between replays, equals the eager call."""
    import sparse_kv_amd as skv

    log("[routed] graph capture of a 4-layer stack, three replays")
    mask, B, Hq, Hkv, d, seq = [1, 0, 0, 1], 2, 8, 2, 128, [64 * 33, 64 * 20 + 7]
    layers, _, L = _stack(54, mask, B, Hq, Hkv, d, seq, 1, 6)
    qs, ks, vs, sl = [x[0] for x in layers], [x[1] for x in layers], [x[2] for x in layers], layers[0][3]
    idx, n = skv.attn_select_topk(None, sl, k=0, n_sink_blocks=1, n_recent_blocks=6, shape=(B, Hkv, L // 64))
    kw = dict(n_shards=8, splits_per_shard=4, sa_block_idx=idx, sa_n_sel=n, sa_splits=8)
    ws = torch.empty(skv.attn_routed_workspace_bytes(qs[0], ks[0], 8, 4, 8), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device="cuda") for _ in qs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        skv.attn_decode_routed(qs, ks, vs, mask, sl, workspace=ws, outs=outs, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        skv.attn_decode_routed(qs, ks, vs, mask, sl, workspace=ws, outs=outs, **kw)
    gen = torch.Generator(device="cpu").manual_seed(7)
    for rep in range(3):
        for q in qs:
            q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype))
        eager = [o.clone() for o in skv.attn_decode_routed(qs, ks, vs, mask, sl, workspace=ws, **kw)]
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(mask)):
            assert torch.equal(outs[i], eager[i]), f"replay {rep} layer {i}"


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


@pytest.mark.parametrize("seed", range(10))
def test_routed_sweep_matches_oracle(seed):
    """A seeded sweep of routed stacks: layer count and route mask, shard and split counts (including
    rows with more than 64 states, merged in two launches), sink and window sizes, group size, head
    dim, ragged rows; sink + window layers poisoned outside their blocks."""
    import sparse_kv_amd as skv

    r = np.random.default_rng(4000 + seed)
    n_layers = int(r.integers(1, 6))
    mask = [int(x) for x in r.integers(0, 2, n_layers)]
    B, Hkv = int(r.integers(1, 4)), int(r.integers(1, 3))
    G, d = int(r.choice([1, 2, 4, 8])), int(r.choice([64, 128]))
    NB = int(r.integers(2, 41))
    seq = [int(x) for x in r.integers(0, 64 * NB + 1, B)]
    seq[0] = 64 * NB
    n_shards, sps, sa_splits = int(r.integers(1, 10)), int(r.integers(1, 9)), int(r.integers(1, 33))
    if seed % 5 == 4:
        n_shards, sps = 9, 8  # 72 states per row
    n_sink, n_recent = int(r.integers(0, 3)), int(r.integers(0, 12))
    log(f"[routed] sweep seed={seed}: mask {mask}, B={B} Hq={G * Hkv} Hkv={Hkv} d={d} seq={seq}, "
        f"{n_shards} shards x {sps} splits, {sa_splits} SA splits, sink {n_sink}, window {n_recent}")
    layers, host, L = _stack(60 + seed, mask, B, G * Hkv, Hkv, d, seq, n_sink, n_recent)
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
