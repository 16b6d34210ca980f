"""GPU parity: ART early-terminated decode (exact stop positions)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.art import art_margin_ok
from tests.gpu_util import TOL, assert_close, log, upload

pytestmark = pytest.mark.gpu

TAU, PHI, P, PROBE = 1e-3, 1e-4, 2, 8


def art_inputs(cfg, B, Hq, Hkv, d, L, seq=None, dtype="bf16", recent=64 * 8, boost=12.0, order=None,
               tau=TAU, phi=PHI, p=P, probe=PROBE):
    """Recency-boosted inputs whose every ART decision clears a 1% band (units redrawn)."""
    attempts = {}
    G = Hq // Hkv
    for _ in range(30):
        inp = synth.make_inputs(cfg, B, Hq, Hkv, d, L, dtype=dtype, kind="recency", seq_lens=seq,
                                attempts=attempts, recent_tokens=recent, boost=boost)
        qf, kf, vf = inp.f64()
        out, stop, traces = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, tau, phi, p, probe, order=order)
        bad = sorted({(b, h // G) for (b, h), tr in traces.items() if not art_margin_ok(tr, tau, phi)})
        if not bad:
            return inp, out, stop
        for u in bad:
            attempts[u] = attempts.get(u, 0) + 1
    raise AssertionError("could not draw inputs with ART decision margins")


# "one": attn_decode_art (one workgroup per (b, kv head)); "ws": attn_decode_art_ws,
# which at these batch sizes spreads each (b, kv head) over several workgroups
PATHS = ["one", "ws"]
# blocks started past the last one needed: the ring of the one-workgroup kernel
# (16 slots), or the shared ring's window, min(128, max(64, folded count))
READ_AHEAD = {"one": lambda need: 16, "ws": lambda need: min(128, max(64, need))}


def run_art(inp, order=None, tau=TAU, phi=PHI, p=P, probe=PROBE, path="one", workspace=None):
    import sparse_kv_amd as skv

    q, k, v, sl = upload(inp)
    o = None if order is None else torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).cuda()
    kw = dict(order=o, tau=tau, phi=phi, patience=p, probe_dim=probe)
    if path == "ws":
        out, stop, fetched = skv.attn_decode_art_ws(q, k, v, sl, workspace=workspace, **kw)
    else:
        out, stop, fetched = skv.attn_decode_art(q, k, v, sl, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), stop.cpu().numpy(), fetched.cpu().numpy()


def check_fetched(fetched, stop, inp, path="one"):
    B, Hq, Hkv, _, _ = inp.shape
    G = Hq // Hkv
    for b in range(B):
        nb = -(-int(inp.seq_lens[b]) // 64)
        for g in range(Hkv):
            need = int(stop[b, g * G:(g + 1) * G].max()) + 1
            assert need <= fetched[b, g] <= min(nb, need + READ_AHEAD[path](need)), (b, g, need, fetched[b, g])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("label,B,Hq,Hkv,d,L,seq,dt", [
    ("bf16-g4-d128", 2, 8, 2, 128, 64 * 48, [64 * 48, 64 * 40 + 17], "bf16"),
    ("bf16-g4-d64", 2, 8, 2, 64, 64 * 40, None, "bf16"),
    ("f32-g1-d64", 1, 2, 2, 64, 64 * 30, None, "f32"),
    ("bf16-g8-d128", 1, 8, 1, 128, 64 * 36, None, "bf16"),
    ("f32-g4-d128", 1, 8, 2, 128, 64 * 30, None, "f32"),
    ("bf16-g6-d64", 2, 12, 2, 64, 64 * 32, [64 * 32, 64 * 27 + 5], "bf16"),
])
def test_art_stop_positions_exact(label, B, Hq, Hkv, d, L, seq, dt, path):
    log(f"[art] {label} ({path})")
    inp, ref_out, ref_stop = art_inputs(40, B, Hq, Hkv, d, L, seq=seq, dtype=dt)
    out, stop, fetched = run_art(inp, path=path)
    log(f"  stops {ref_stop.ravel().tolist()}")
    assert np.array_equal(stop, ref_stop), (stop, ref_stop)
    assert_close(out, ref_out, TOL, "ART output")
    check_fetched(fetched, stop, inp, path)
    assert (ref_stop < np.array([-(-int(s) // 64) for s in inp.seq_lens])[:, None] - 1).any(), \
        "the case should stop early somewhere"


@pytest.mark.parametrize("path", PATHS)
def test_art_special_cases_reduce_to_dense(path):
    log(f"[art] tau = phi = 0, probe off, patience > nb, tau = phi = inf ({path})")
    inp = synth.make_inputs(41, 2, 8, 2, 128, 64 * 20, kind="recency", seq_lens=[64 * 20, 64 * 11 + 5],
                            recent_tokens=64 * 4)
    qf, kf, vf = inp.f64()
    dense = oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale)
    nbs = np.array([20, 12])[:, None]
    for tau, phi, p, probe in ((0.0, 0.0, 1, 8), (1.0, 1.0, 2, 0), (math.inf, math.inf, 30, 8)):
        out, stop, fetched = run_art(inp, tau=tau, phi=phi, p=p, probe=probe, path=path)
        assert (stop == nbs - 1).all(), (tau, phi, p, probe, stop)
        assert (fetched == nbs).all()
        assert_close(out, dense, TOL, f"dense-equivalent ART tau={tau} probe={probe}")
    out, stop, fetched = run_art(inp, tau=math.inf, phi=math.inf, p=1, probe=8, path=path)
    assert (stop == 1).all()
    ref_out, ref_stop, _ = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, math.inf, math.inf, 1, 8)
    assert_close(out, ref_out, TOL, "stop after two blocks")


@pytest.mark.parametrize("path", PATHS)
def test_art_custom_visit_order(path):
    log(f"[art] custom visit orders starting with block 0 ({path})")
    B, Hq, Hkv, L = 1, 8, 2, 64 * 24
    nb = 24
    r = np.random.default_rng(3)
    order = np.zeros((B, Hkv, nb), dtype=np.int32)
    for g in range(Hkv):
        order[0, g] = [0] + list(r.permutation(np.arange(1, nb)))
    inp = synth.make_inputs(42, B, Hq, Hkv, 128, L, kind="recency", recent_tokens=64 * 6)
    qf, kf, vf = inp.f64()
    out, stop, _ = run_art(inp, order=order, tau=0.0, phi=0.0, path=path)
    assert (stop == nb - 1).all()
    assert_close(out, oracle.decode_dense(qf, kf, vf, inp.seq_lens, inp.scale), TOL, "order-invariant dense")
    inp, ref_out, ref_stop = art_inputs(43, B, Hq, Hkv, 128, L, recent=64 * 6, order=order)
    out, stop, _ = run_art(inp, order=order, path=path)
    assert np.array_equal(stop, ref_stop)
    assert_close(out, ref_out, TOL, "custom-order ART output")


@pytest.mark.parametrize("path", PATHS)
def test_art_empty_and_single_block_rows(path):
    log(f"[art] rows with 0 and 1 blocks ({path})")
    inp = synth.make_inputs(44, 3, 4, 1, 128, 64 * 4, kind="gauss", seq_lens=[0, 30, 64 * 4])
    out, stop, fetched = run_art(inp, path=path)
    qf, kf, vf = inp.f64()
    ref_out, ref_stop, _ = oracle.art_decode(qf, kf, vf, inp.seq_lens, inp.scale, TAU, PHI, P, PROBE)
    assert stop[0].tolist() == [-1] * 4 and not out[0].any() and fetched[0, 0] == 0
    assert stop[1].tolist() == [0] * 4 and fetched[1, 0] == 1
    assert np.array_equal(stop, ref_stop)
    assert_close(out, ref_out, TOL, "output")


def test_art_workspace_reused_across_calls():
    """One workspace, three calls in a row (G = 4, then G = 8 with a smaller
    batch, then G = 4 again): every call starts from a clean ring."""
    import sparse_kv_amd as skv

    log("[art] workspace reuse")
    cases = [(45, 2, 8, 2, [64 * 30, 64 * 22 + 9]), (46, 1, 8, 1, [64 * 26]), (47, 2, 8, 2, [64 * 25, 64 * 30])]
    need = max(skv.attn_art_workspace_bytes(torch.empty(B, Hq, 128, dtype=torch.bfloat16),
                                            torch.empty(B, Hkv, 64 * 30, 128, dtype=torch.bfloat16))
               for _, B, Hq, Hkv, _ in cases)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0x7f)  # contents from an earlier user must not matter
    for seed, B, Hq, Hkv, seq in cases:
        inp, ref_out, ref_stop = art_inputs(seed, B, Hq, Hkv, 128, 64 * 30, seq=seq)
        out, stop, fetched = run_art(inp, path="ws", workspace=ws)
        assert np.array_equal(stop, ref_stop), (seed, stop, ref_stop)
        assert_close(out, ref_out, TOL, f"ART output, seed {seed}")
        check_fetched(fetched, stop, inp, "ws")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("probe", [1, 3, 12, 16])
def test_art_probe_widths(probe, path):
    # probes narrower than 8 channels, and wider ones (the scan then carries 16)
    log(f"[art] probe_dim = {probe} ({path})")
    inp, ref_out, ref_stop = art_inputs(41, 2, 8, 2, 128, 64 * 40, seq=[64 * 40, 64 * 33 + 9], probe=probe)
    out, stop, fetched = run_art(inp, probe=probe, path=path)
    log(f"  stops {ref_stop.ravel().tolist()}")
    assert np.array_equal(stop, ref_stop), (stop, ref_stop)
    assert_close(out, ref_out, TOL, f"ART output, probe {probe}")
    check_fetched(fetched, stop, inp, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("p", [1, 3, 5])
def test_art_patience(p, path):
    # the stop needs p consecutive stable steps ("ART" summary, §2.3)
    log(f"[art] patience {p} ({path})")
    inp, ref_out, ref_stop = art_inputs(42, 2, 8, 2, 128, 64 * 40, seq=[64 * 40, 64 * 31 + 3], p=p)
    out, stop, fetched = run_art(inp, p=p, path=path)
    log(f"  stops {ref_stop.ravel().tolist()}")
    assert np.array_equal(stop, ref_stop), (stop, ref_stop)
    assert_close(out, ref_out, TOL, f"ART output, patience {p}")
    check_fetched(fetched, stop, inp, path)


@pytest.mark.parametrize("B", [12, 16])
def test_art_across_workgroups_at_many_units(B):
    # 96 and 128 (b, kv head) units: two workgroups per unit on a 256-CU device (four at the smaller
    # sizes above), and 128 is the largest count the workspace form spreads
    log(f"[art] {B * 8} units through attn_decode_art_ws")
    inp, ref_out, ref_stop = art_inputs(43, B, 32, 8, 128, 64 * 20, recent=64 * 6)
    import sparse_kv_amd as skv

    need = skv.attn_art_workspace_bytes(torch.empty(B, 32, 128, dtype=torch.bfloat16),
                                        torch.empty(B, 8, 64 * 20, 128, dtype=torch.bfloat16))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 1, "the workspace form should be available at this unit count"
    out, stop, fetched = run_art(inp, path="ws", workspace=ws)
    assert np.array_equal(stop, ref_stop), (stop, ref_stop)
    assert_close(out, ref_out, TOL, f"ART output, {B * 8} units")
    check_fetched(fetched, stop, inp, "ws")
