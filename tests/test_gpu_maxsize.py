"""GPU parity at the size limits: a (b, kv head) K/V slice of exactly 2 GiB
(131072 blocks of bf16 d 128, the largest the library accepts) and top-k rows
longer than the candidates a workgroup stages in LDS; a paged pool whose blocks
all lie past byte offset 2^32.

The 2 GiB slice is built on the device: zero keys and values except a few
tokens, so the exact attention output has a closed form (softmax attention
as defined in the "ART (Attention Run-time Termination)" summary, §2.1): with
logits s_t, the output is sum_t e^{s_t} v_t / sum_t e^{s_t}, where every
token with a zero key adds e^0 = 1 to the denominator and nothing to the
numerator unless its value row is set."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, assert_close, log, upload

pytestmark = pytest.mark.gpu

D = 128
NB = 131072  # 131072 blocks x 64 tokens x 256 bytes = 2 GiB per K (and V) slice
N = NB * 64


def bf16_round(x):
    return float(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).float())


def build_max_slice():
    """Keys: zero except channel 0 of three tokens; values: zero except a few
    rows.  Returns device q, k, v and the host description."""
    scale = 1.0 / math.sqrt(D)
    qv = 8.0
    special = {0: 19.0, N // 2 + 37: 18.0, N - 1: 20.0}  # token -> target logit
    key0 = {t: bf16_round(s / (scale * qv)) for t, s in special.items()}
    r = np.random.default_rng(123)
    vrows = sorted({0, 1, N // 2 + 37, N - 65, N - 2, N - 1})
    vals = {t: r.standard_normal(D).astype(np.float32) for t in vrows}
    q = torch.zeros(1, 1, D, dtype=torch.bfloat16, device="cuda")
    q[0, 0, 0] = qv
    k = torch.zeros(1, 1, N, D, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(1, 1, N, D, dtype=torch.bfloat16, device="cuda")
    for t, a in key0.items():
        k[0, 0, t, 0] = a
    for t, x in vals.items():
        v[0, 0, t] = torch.from_numpy(x).to(torch.bfloat16)
    vals = {t: v[0, 0, t].float().cpu().numpy().astype(np.float64) for t in vrows}  # the stored bf16 rows
    return q, k, v, dict(scale=scale, qv=qv, key0=key0, vals=vals)


def exact_output(desc, tokens_lo_hi):
    """Closed-form attention over the token ranges [(lo, hi), ...]."""
    n_tok = sum(hi - lo for lo, hi in tokens_lo_hi)
    inside = lambda t: any(lo <= t < hi for lo, hi in tokens_lo_hi)
    logits = {t: desc["scale"] * desc["qv"] * a for t, a in desc["key0"].items() if inside(t)}
    M = max(list(logits.values()) + [0.0])
    num = np.zeros(D)
    den = (n_tok - len(logits)) * math.exp(-M)
    for t, s in logits.items():
        den += math.exp(s - M)
    for t, x in desc["vals"].items():
        if inside(t):
            num += math.exp(logits.get(t, 0.0) - M) * x
    return num / den


@pytest.fixture(scope="module")
def max_slice():
    q, k, v, desc = build_max_slice()
    torch.cuda.synchronize()
    yield q, k, v, desc
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("L", [N, N - 30, 64 * (NB // 2) + 1])
def test_dense_decode_on_a_2gib_slice(max_slice, L):
    import sparse_kv_amd as skv

    q, k, v, desc = max_slice
    log(f"[max] dense decode over a 2 GiB K/V slice, L={L}")
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    want = exact_output(desc, [(0, L)])
    for S in (1, 4, 64):
        out = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, sl, num_splits=S))
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[0, 0], want, TOL, f"L={L} S={S}")


def test_listed_decode_on_a_2gib_slice(max_slice):
    import sparse_kv_amd as skv

    q, k, v, desc = max_slice
    log("[max] listed-block decode over blocks 0, the middle one and the last of a 2 GiB slice")
    blocks = [0, (N // 2 + 37) // 64, NB - 1]
    idx = torch.tensor([[blocks]], dtype=torch.int32, device="cuda")
    n = torch.tensor([[len(blocks)]], dtype=torch.int32, device="cuda")
    want = exact_output(desc, [(64 * j, 64 * j + 64) for j in blocks])
    for S in (1, 3):
        out = skv.attn_merge_states(*skv.attn_decode_sparse(q, k, v, idx, n, None, num_splits=S))
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[0, 0], want, TOL, f"listed S={S}")


@pytest.mark.parametrize("NBr", [20000, 40001])
def test_topk_rows_longer_than_the_staged_keys(NBr):
    # more candidates than the 16384 keys a workgroup stages: every select pass reads memory
    import sparse_kv_amd as skv

    log(f"[max] top-k on {NBr}-block rows")
    r = np.random.default_rng(NBr)
    B, Hkv = 1, 2
    s = (r.standard_normal((B, Hkv, NBr)) * 2).astype(np.float32)
    s[0, 1] = np.round(s[0, 1] * 8) / 8  # heavy ties
    s[0, 0, 5000:5100] = s[0, 0, 777]
    seq = np.array([64 * NBr - 5], dtype=np.int32)
    for k, ns, nr in ((1, 1, 0), (2000, 1, 64), (NBr // 2, 0, 0), (NBr, 1, 64)):
        idx, n = skv.attn_select_topk(torch.from_numpy(s).cuda(), torch.from_numpy(seq).cuda(), k=k,
                                      n_sink_blocks=ns, n_recent_blocks=nr)
        torch.cuda.synchronize()
        idx, n = idx.cpu().numpy(), n.cpu().numpy()
        ref = oracle.select_all(s.astype(np.float64), seq, k, ns, nr)
        for g in range(Hkv):
            assert n[0, g] == len(ref[0][g]), (k, g)
            assert idx[0, g, :n[0, g]].tolist() == ref[0][g], (k, g)


@pytest.mark.parametrize("path", ["one", "ws"])
def test_art_on_a_2gib_slice(max_slice, path):
    # two properties that hold at any size ("ART" summary, §2.2-2.3): tau = phi = 0 never stops, so ART
    # folds all 131072 blocks and equals dense attention; tau = phi = inf with p = 1 stops at visit
    # position 1, after block 0 and the newest block
    import sparse_kv_amd as skv

    q, k, v, desc = max_slice
    log(f"[max] ART over a 2 GiB slice ({path})")
    ws = torch.empty(max(skv.attn_art_workspace_bytes(q, k), 1), dtype=torch.uint8, device="cuda")
    run = (lambda **kw: skv.attn_decode_art_ws(q, k, v, None, workspace=ws, **kw)) if path == "ws" else \
        (lambda **kw: skv.attn_decode_art(q, k, v, None, **kw))
    out, stop, fetched = run(tau=0.0, phi=0.0, patience=2, probe_dim=8)
    torch.cuda.synchronize()
    assert int(stop[0, 0]) == NB - 1 and int(fetched[0, 0]) == NB
    assert_close(out.cpu().numpy()[0, 0], exact_output(desc, [(0, N)]), TOL, f"ART tau=phi=0 ({path})")
    out, stop, fetched = run(tau=math.inf, phi=math.inf, patience=1, probe_dim=8)
    torch.cuda.synchronize()
    assert int(stop[0, 0]) == 1
    assert_close(out.cpu().numpy()[0, 0], exact_output(desc, [(0, 64), (N - 64, N)]), TOL,
                 f"ART tau=phi=inf p=1 ({path})")


def test_paged_pool_past_4gib():
    # pool runs placed past byte offset 2^32 of the pool: the per-block offsets need 64 bits
    import sparse_kv_amd as skv
    import synth

    log("[max] paged decode with every block stored past 4 GiB into the pool")
    B, Hq, Hkv, d, NBl = 2, 8, 2, 128, 40
    inp = synth.make_inputs(77, B, Hq, Hkv, d, 64 * NBl, kind="gauss", seq_lens=[64 * NBl, 64 * 23 + 7])
    q, k, v, sl = upload(inp)
    P = 140000  # 140000 x 2 heads x 16 KiB = 4.6 GB per pool
    first = (1 << 32) // (Hkv * 64 * d * 2) + 11  # first slot whose offset is past 2^32
    assert first + B * NBl < P
    perm = torch.randperm(B * NBl, generator=torch.Generator().manual_seed(3)) + first
    table = perm.view(B, NBl).to(torch.int32).cuda()
    kp = torch.full((P, Hkv, 64, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full((P, Hkv, 64, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb = k.view(B, Hkv, NBl, 64, d).permute(0, 2, 1, 3, 4).reshape(B * NBl, Hkv, 64, d)
    vb = v.view(B, Hkv, NBl, 64, d).permute(0, 2, 1, 3, 4).reshape(B * NBl, Hkv, 64, d)
    kp[table.view(-1).long()] = kb
    vp[table.view(-1).long()] = vb
    qf, kf, vf = inp.f64()
    ref = oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale)
    out = skv.attn_merge_states(*skv.attn_decode_dense_paged(q, kp, vp, table, sl, num_splits=3))
    contiguous = skv.attn_merge_states(*skv.attn_decode_dense(q, k, v, sl, num_splits=3))
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, TOL, "dense over a pool past 4 GiB")
    assert torch.equal(out, contiguous), "paged and contiguous dense outputs differ"
    ao, astop, _ = skv.attn_decode_art_paged(q, kp, vp, table, sl, tau=0.0, phi=0.0, patience=2, probe_dim=8)
    torch.cuda.synchronize()
    assert (astop.cpu().numpy() == np.array([[NBl - 1] * Hq, [23] * Hq])).all()
    assert_close(ao.cpu().numpy(), ref, TOL, "ART (tau = phi = 0) over a pool past 4 GiB")
    del kp, vp
    torch.cuda.empty_cache()
