"""GPU test of attn_decode_routed_static, the routed entry point that allocates
nothing: through the C ABI its outputs equal attn_decode_routed's (same
kernels, the states in the library's static scratch instead of a caller
workspace), on two calls in a row -- the second smaller, on another stream --
and a call whose states would not fit the scratch is refused on the host."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TOL, assert_close, log, upload

pytestmark = pytest.mark.gpu


def stack(cfg, n_layers, B, Hq, Hkv, d, L, seq, mask, n_sink, n_recent):
    layers, host = [], []
    lists = []
    for b in range(B):
        nb = -(-seq[b] // 64)
        lists.append([sorted(oracle.selection.forced_blocks(nb, n_sink, n_recent))] * Hkv)
    for i in range(n_layers):
        inp = synth.make_inputs(cfg, B, Hq, Hkv, d, L, kind="needles", seq_lens=seq, layer=i)
        host.append(inp.f64())
        if not mask[i]:
            synth.poison_blocks(inp, lists)
        layers.append(upload(inp))
    return layers, host, lists


def test_routed_static_matches_routed_on_two_calls():
    import sparse_kv_amd as skv

    cases = [
        # (cfg, mask, B, Hq, Hkv, d, L, seq, shards, splits per shard, SA splits, sink, recent)
        (70, [1, 0, 1, 0], 2, 8, 2, 128, 64 * 40, [64 * 40, 64 * 29 + 3], 8, 2, 3, 1, 6),
        (71, [0, 1], 1, 8, 2, 64, 64 * 12, [64 * 12 - 5], 2, 3, 2, 1, 3),
    ]
    side = torch.cuda.Stream()
    for i, (cfg, mask, B, Hq, Hkv, d, L, seq, ns, sps, sas, n_sink, n_recent) in enumerate(cases):
        log(f"[no-alloc] call {i + 1}: {len(mask)} layers {mask}, B {B}, d {d}, L {L}, {ns} x {sps} splits")
        layers, host, lists = stack(cfg, len(mask), B, Hq, Hkv, d, L, seq, mask, n_sink, n_recent)
        sl = layers[0][3]
        sa_idx, sa_n = skv.attn_select_topk(None, sl, k=0, n_sink_blocks=n_sink, n_recent_blocks=n_recent,
                                            shape=(B, Hkv, L // 64), device="cuda")
        qs, ks, vs = ([x[j] for x in layers] for j in range(3))
        kw = dict(n_shards=ns, splits_per_shard=sps, sa_block_idx=sa_idx, sa_n_sel=sa_n, sa_splits=sas)
        ref = skv.attn_decode_routed(qs, ks, vs, mask, sl, **kw)
        outs = [torch.full((B, Hq, d), float("nan"), device="cuda") for _ in mask]
        torch.cuda.synchronize()
        stream = side if i == 1 else torch.cuda.current_stream()
        with torch.cuda.stream(stream):
            skv.attn_decode_routed_static(qs, ks, vs, mask, sl, outs=outs, **kw)
        torch.cuda.synchronize()
        want = oracle.routed_layer_outputs(host, seq, 1 / np.sqrt(d), mask, n_sink, n_recent)
        for j in range(len(mask)):
            got, r = outs[j].cpu().numpy(), ref[j].cpu().numpy()
            assert np.isfinite(got).all()
            assert_close(got, r, TOL, f"layer {j}: static vs workspace entry point")
            assert np.array_equal(got, r), f"layer {j}: same kernels, same splits -> identical outputs"
            assert_close(got, want[j], TOL, f"layer {j}: static entry point vs oracle")


def test_routed_static_refuses_states_beyond_the_scratch():
    import sparse_kv_amd as skv

    # 64 x 32 query rows x 32 splits x 128 channels of states: 32 MiB > the 8 MiB scratch
    B, Hq, Hkv, d, L = 64, 32, 8, 128, 64
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, L, d), dtype=torch.bfloat16, device="cuda")
    need = skv.attn_routed_workspace_bytes(q, k, 8, 4, 4)
    assert need > skv.ROUTED_STATIC_BYTES
    with pytest.raises(ValueError, match="workspace too small"):
        skv.attn_decode_routed_static([q], [k], [k], [1], None, n_shards=8, splits_per_shard=4)
    # the same stack with fewer splits fits and runs
    out = skv.attn_decode_routed_static([q], [k], [k], [1], None, n_shards=1, splits_per_shard=1)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0]).all() and not out[0].any()
