"""GPU: a whole decode step (dense + merge, scores + top-k + listed-block decode
+ merge, ART across workgroups, sink + window) captured once in a HIP graph and
replayed with new query data each time; every replay must equal the eager
calls on the same data bit for bit (the library queues no memset and
allocates nothing inside the calls that take their outputs and workspaces,
and every entry point, the multi-workgroup ART included, is reproducible)."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import log, upload

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    import sparse_kv_amd as skv

    log("[graph] capture one decode step, replay with new queries")
    B, Hq, Hkv, d, L = 2, 8, 2, 128, 64 * 40
    inp = synth.make_inputs(60, B, Hq, Hkv, d, L, kind="mixture", seq_lens=[L, 64 * 33 + 5])
    q, k, v, sl = upload(inp)
    NB = L // 64
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    S = 3
    st = [(torch.empty((B, Hq, S), **f32), torch.empty((B, Hq, S), **f32), torch.empty((B, Hq, S, d), **f32))
          for _ in range(3)]
    C = skv.attn_build_centroids(k, sl)
    scores = torch.empty((B, Hkv, NB), **f32)
    max_sel = 1 + 4 + 6
    sel = torch.empty((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    nsel = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    win, nwin = skv.attn_select_topk(None, sl, k=0, n_sink_blocks=1, n_recent_blocks=8, shape=(B, Hkv, NB),
                                     device=dev)
    ws = torch.empty(skv.attn_art_workspace_bytes(q, k), dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, Hq, d), **f32) for _ in range(4)]
    stop = torch.empty((B, Hq), dtype=torch.int32, device=dev)

    def step():
        skv.attn_decode_dense(q, k, v, sl, num_splits=S, m=st[0][0], l=st[0][1], o=st[0][2])
        skv.attn_merge_states(*st[0], out=outs[0])
        skv.attn_score_centroids(q, C, sl, out=scores)
        skv.attn_select_topk(scores, sl, k=6, n_sink_blocks=1, n_recent_blocks=4, max_sel=max_sel, block_idx=sel,
                             n_sel=nsel)
        skv.attn_decode_sparse(q, k, v, sel, nsel, sl, num_splits=S, m=st[1][0], l=st[1][1], o=st[1][2])
        skv.attn_merge_states(*st[1], out=outs[1])
        skv.attn_decode_art_ws(q, k, v, sl, tau=2e-2, phi=2e-3, patience=2, probe_dim=8, workspace=ws,
                               out=outs[2], stop_pos=stop)
        skv.attn_decode_sparse(q, k, v, win, nwin, sl, num_splits=S, m=st[2][0], l=st[2][1], o=st[2][2])
        skv.attn_merge_states(*st[2], out=outs[3])

    def snapshot():
        return [o.clone() for o in outs] + [stop.clone(), sel.clone(), nsel.clone()]

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    r = np.random.default_rng(61)
    for rep in range(3):
        newq = torch.from_numpy(r.standard_normal(q.shape).astype(np.float32)).to(dev).to(q.dtype)
        q.copy_(newq)
        step()  # eager on the new query
        torch.cuda.synchronize()
        want = snapshot()
        for o in outs:
            o.fill_(float("nan"))
        stop.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), (rep, i, float((a.float() - b.float()).abs().max()))
