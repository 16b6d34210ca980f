"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""

import math
import sys

import numpy as np
import torch

import synth


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def upload(inp: synth.DecodeInputs, device="cuda"):
    q = to_dev(inp.q, inp.dtype, device)
    k = to_dev(inp.k, inp.dtype, device)
    v = to_dev(inp.v, inp.dtype, device)
    seq = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device)
    return q, k, v, seq


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def assert_close(got, ref, tol, what):
    err = max_abs(got, ref)
    log(f"  {what}: max-abs error {err:.3e} (tolerance {tol:.1e})")
    assert np.isfinite(np.asarray(got)).all(), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max-abs error {err} > {tol}"
    return err


def assert_states_close(m, l, o, rm, rl, ro, tol_o, what):
    """Split states: empty splits must be (-inf, 0, 0); others close."""
    m, l, o = (x.detach().cpu().numpy().astype(np.float64) for x in (m, l, o))
    empty = rl == 0
    assert np.array_equal(l == 0, empty), f"{what}: empty-split pattern differs"
    assert np.all(np.isneginf(m[empty])) and not o[empty].any(), f"{what}: empty splits not (-inf, 0, 0)"
    full = ~empty
    if full.any():
        em = float(np.max(np.abs(m[full] - rm[full]) / np.maximum(1.0, np.abs(rm[full]))))
        el = float(np.max(np.abs(l[full] - rl[full]) / rl[full]))
        log(f"  {what}: m rel {em:.2e}, l rel {el:.2e}")
        assert em < 1e-4 and el < 1e-4, f"{what}: m/l mismatch ({em}, {el})"
    assert_close(o, ro, tol_o, what + " o")


TOL = 5e-3  # max-abs output tolerance against the float64 oracle
