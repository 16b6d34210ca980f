"""GPU parity: top-k selection over a seeded sweep of shapes and score patterns.

Each case draws a row length (either side of the 2048-block switch between
the register-resident and the LDS-staged kernel, and of the 256-block round
size), k, the sink and recent counts, sequence lengths (empty, partial last
block, full) and a score pattern: continuous, coarsely quantised (heavy ties,
so the k-th key's histogram bin overflows into the radix select), all equal,
or tightly clustered in one 12-bit bin.  Indices and counts must equal the
oracle's exactly, and every entry past the count must be -1.  A second sweep
does the same for two-level selection from the query (super-block group
sizes 2-16, k_coarse from none to all, ragged rows, both dtypes), on inputs
redrawn until both decision boundaries clear a 1e-4 score gap.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

ROW_LENGTHS = [1, 2, 17, 255, 256, 257, 1000, 2047, 2048, 2049, 3000, 4096]
PATTERNS = ["normal", "quantised", "equal", "clustered"]


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    NB = int(ROW_LENGTHS[seed % len(ROW_LENGTHS)])
    pattern = PATTERNS[(seed // len(ROW_LENGTHS)) % len(PATTERNS)]
    B, Hkv = int(r.integers(1, 4)), int(r.integers(1, 4))
    k = int(r.choice([0, 1, int(r.integers(0, NB + 1)), NB // 10, NB, NB + 3]))
    ns, nr = int(r.integers(0, 4)), int(r.choice([0, 1, int(r.integers(0, 80))]))
    if pattern == "normal":
        s = r.standard_normal((B, Hkv, NB))
    elif pattern == "quantised":
        s = r.integers(0, 5, (B, Hkv, NB)) / 4.0
    elif pattern == "equal":
        s = np.full((B, Hkv, NB), 0.5)
    else:
        s = 1.0 + r.integers(0, 4000, (B, Hkv, NB)) * 1e-7
    s = s.astype(np.float32)
    if NB > 3:
        s[0, 0, 1] = -0.0
        s[0, 0, 2] = 0.0
    seq = r.integers(0, NB * 64 + 1, B).astype(np.int32)
    seq[0] = NB * 64
    max_sel = min(NB, ns + nr + k) + int(r.integers(0, 3))
    return NB, pattern, B, Hkv, k, ns, nr, s, seq, max(max_sel, 1)


@pytest.mark.parametrize("seed", range(48))
def test_topk_sweep_matches_oracle(seed):
    import sparse_kv_amd as skv

    NB, pattern, B, Hkv, k, ns, nr, s, seq, max_sel = _case(seed)
    log(f"[select-sweep] seed={seed} NB={NB} {pattern} B={B} Hkv={Hkv} k={k} sink={ns} recent={nr} max_sel={max_sel}")
    scores = torch.from_numpy(s).cuda() if k > 0 else None
    idx, n = skv.attn_select_topk(scores, torch.from_numpy(seq).cuda(), k=k, n_sink_blocks=ns, n_recent_blocks=nr,
                                  max_sel=max_sel, shape=(B, Hkv, NB), device="cuda")
    torch.cuda.synchronize()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    ref = oracle.select_all(s.astype(np.float64), seq, k, ns, nr)
    for b in range(B):
        for g in range(Hkv):
            want = ref[b][g][:max_sel]
            assert n[b, g] == len(want), (b, g, int(n[b, g]), len(want))
            assert idx[b, g, :len(want)].tolist() == want, (b, g)
            assert (idx[b, g, len(want):] == -1).all(), (b, g)


def _two_level_case(seed):
    r = np.random.default_rng(3000 + seed)
    B, Hkv = int(r.integers(1, 3)), int(r.integers(1, 3))
    G = int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    dt = str(r.choice(["bf16", "f32"]))
    NB = int(r.integers(4, 65))
    L = 64 * NB
    seq = [int(x) for x in r.integers(1, L + 1, B)]
    seq[0] = L
    group = int(r.choice([2, 3, 4, 8, 16]))
    kc = int(r.choice([0, 1, 2, int(r.integers(1, 9)), 100]))
    k = int(r.integers(0, 3 * group + 1))
    ns, nr = int(r.integers(0, 3)), int(r.integers(0, 6))
    return B, Hkv, G, d, dt, L, seq, group, kc, k, ns, nr


@pytest.mark.parametrize("seed", range(16))
def test_two_level_sweep_matches_oracle(seed):
    import sparse_kv_amd as skv
    from tests.gpu_util import upload
    from tests.test_gpu_select import two_level_inputs

    B, Hkv, G, d, dt, L, seq, group, kc, k, ns, nr = _two_level_case(seed)
    log(f"[select-sweep] two-level seed={seed} B={B} Hq={Hkv * G} Hkv={Hkv} d={d} {dt} L={L} seq={seq} "
        f"group={group} k_coarse={kc} k={k} sink={ns} recent={nr}")
    inp, lists = two_level_inputs(90 + seed, B, Hkv * G, Hkv, d, L, seq, group, kc, k, ns, nr, dtype=dt)
    q, kk, _, sl = upload(inp)
    C = skv.attn_build_centroids(kk, sl)
    C2 = skv.attn_build_super_centroids(C, group, sl)
    idx, n = skv.attn_select_two_level(q, C, C2, group, sl, k_coarse=kc, k=k, n_sink_blocks=ns, n_recent_blocks=nr)
    torch.cuda.synchronize()
    idx, n = idx.cpu().numpy(), n.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            assert n[b, g] == len(lists[b][g]), (b, g, int(n[b, g]), lists[b][g])
            assert idx[b, g, :n[b, g]].tolist() == lists[b][g], (b, g)
            assert (idx[b, g, n[b, g]:] == -1).all(), (b, g)
