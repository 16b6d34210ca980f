"""Seeded synthetic decode-attention inputs, shared by the tests, the benchmark
and the smoke check.

This module holds no attention arithmetic: it only draws random tensors with
the shapes and value structure of the workloads (Llama-3.1-8B / Qwen3-8B
shaped decode layers over a block-organised KV cache) and encodes them as
bf16 or fp32.  Both the HIP library and the CPU oracle consume exactly these
values (the oracle through an exact float64 upcast).

Random streams: ``numpy.random.default_rng(SeedSequence([0x5EED, cfg, tensor,
layer, b, kvh, attempt]))``; every (batch row, KV head) unit is drawn on its
own, so any unit can be regenerated (``attempt`` > 0 redraws one unit) and
large inputs are produced in parallel threads.

Value recipes (readings of the workload descriptions):

* ``gauss``: Q, K, V ~ N(0, 1).
* ``needles``: as ``gauss`` plus, per unit, ``n_needles`` key positions drawn
  uniformly without replacement outside block 0 whose keys are
  4 * u + N(0, I), u = unit vector of the sum of the group's query heads.
* ``mixture``: block-coherent Gaussian mixture keys: per unit 256 centres
  mu_c ~ N(0, I), one centre z_j per 64-token block, k_t = mu_{z_j} + 0.3 eps.
* ``recency``: as ``gauss`` plus k_t += 12 * u for the last 4096 valid tokens.

Tokens at or beyond a sequence's length hold NaN (bf16 0x7FC0 / fp32 NaN) so
that any read past the end poisons the result.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

SEED_ROOT = 0x5EED
T_Q, T_K, T_V, T_MIX, T_NEEDLE, T_ROUTE, T_LEN = range(7)
BF16_NAN = np.uint16(0x7FC0)
BLOCK = 64


def rng_for(cfg: int, tensor: int, layer: int = 0, b: int = 0, kvh: int = 0, attempt: int = 0):
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg, tensor, layer, b, kvh, attempt]))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class DecodeInputs:
    """One decode step's inputs.

    q [B, Hq, d]; k, v [B, Hkv, Lmax, d]; bf16 tensors are uint16 bit
    patterns, fp32 tensors are float32.  seq_lens int32 [B].
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seq_lens: np.ndarray
    dtype: str

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.q.shape[-1])

    @property
    def shape(self):
        B, Hq, d = self.q.shape
        return B, Hq, self.k.shape[1], d, self.k.shape[2]

    def upcast(self, a: np.ndarray) -> np.ndarray:
        """Exact float64 copy of one of the stored tensors."""
        if self.dtype == "bf16":
            return bf16_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float32).astype(np.float64)

    def f64(self):
        return self.upcast(self.q), self.upcast(self.k), self.upcast(self.v)

    def unit_f64(self, b: int, g: int):
        """float64 (q of the group [G, d], K [Lmax, d], V [Lmax, d]) of one unit."""
        G = self.q.shape[1] // self.k.shape[1]
        return (self.upcast(self.q[b, g * G:(g + 1) * G]), self.upcast(self.k[b, g]),
                self.upcast(self.v[b, g]))


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _decode(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(x) if dtype == "bf16" else x


def _unit_direction(q_group_encoded: np.ndarray, dtype: str) -> np.ndarray:
    s = _decode(q_group_encoded, dtype).astype(np.float64).sum(axis=0)
    n = np.linalg.norm(s)
    return (s / n) if n > 0 else np.eye(len(s))[0]


def draw_unit(cfg: int, b: int, g: int, G: int, d: int, L: int, Lb: int, dtype: str = "bf16",
              kind: str = "gauss", layer: int = 0, attempt: int = 0, n_needles: int = 16,
              n_clusters: int = 256, sigma_within: float = 0.3, recent_tokens: int = 4096,
              boost: float = 12.0, pad_nan: bool = True):
    """Draw one (batch row b, KV head g) unit: (q of the group [G, d], K [L, d], V [L, d]),
    encoded (bf16 bit patterns or float32).  Lb is the row's sequence length; tokens at or
    beyond it hold NaN when pad_nan.  make_inputs assembles a batch from exactly these."""
    qg = _encode(rng_for(cfg, T_Q, layer, b, g, attempt).standard_normal((G, d), dtype=np.float32), dtype)
    rk = rng_for(cfg, T_K, layer, b, g, attempt)
    if kind == "mixture":
        rm = rng_for(cfg, T_MIX, layer, b, g, attempt)
        mu = rm.standard_normal((n_clusters, d), dtype=np.float32)
        nblk = -(-L // BLOCK)
        z = rm.integers(0, n_clusters, size=nblk)
        kk = rk.standard_normal((L, d), dtype=np.float32) * np.float32(sigma_within)
        kk += np.repeat(mu[z], BLOCK, axis=0)[:L]
    else:
        kk = rk.standard_normal((L, d), dtype=np.float32)
    if kind in ("needles", "recency") and Lb > 0:
        u = _unit_direction(qg, dtype).astype(np.float32)
        if kind == "needles" and Lb > BLOCK:
            rn = rng_for(cfg, T_NEEDLE, layer, b, g, attempt)
            n = min(n_needles, Lb - BLOCK)
            pos = BLOCK + rn.choice(Lb - BLOCK, size=n, replace=False)
            kk[pos] = np.float32(4.0) * u + rn.standard_normal((n, d), dtype=np.float32)
        if kind == "recency":
            lo = max(0, Lb - recent_tokens)
            kk[lo:Lb] += np.float32(boost) * u
    k = _encode(kk, dtype)
    del kk
    v = _encode(rng_for(cfg, T_V, layer, b, g, attempt).standard_normal((L, d), dtype=np.float32), dtype)
    if pad_nan and Lb < L:
        nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
        k[Lb:] = nan
        v[Lb:] = nan
    return qg, k, v


def make_inputs(cfg: int, B: int, Hq: int, Hkv: int, d: int, L: int, dtype: str = "bf16",
                kind: str = "gauss", seq_lens=None, layer: int = 0, attempts=None,
                threads: int | None = None, n_needles: int = 16, n_clusters: int = 256,
                sigma_within: float = 0.3, recent_tokens: int = 4096, boost: float = 12.0,
                pad_nan: bool = True) -> DecodeInputs:
    """Draw one decode step's inputs.

    L is the allocated length Lmax; seq_lens (default: all L) may be ragged.
    attempts: optional dict {(b, kvh): attempt} to redraw chosen units.
    """
    assert Hq % Hkv == 0 and dtype in ("bf16", "f32")
    G = Hq // Hkv
    seq = np.full(B, L, dtype=np.int32) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    assert seq.shape == (B,) and (seq >= 0).all() and (seq <= L).all()
    store = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((B, Hq, d), dtype=store)
    k = np.empty((B, Hkv, L, d), dtype=store)
    v = np.empty((B, Hkv, L, d), dtype=store)
    attempts = attempts or {}

    def unit(bg):
        b, g = bg
        qg, kk, vv = draw_unit(cfg, b, g, G, d, L, int(seq[b]), dtype, kind, layer, attempts.get((b, g), 0),
                               n_needles, n_clusters, sigma_within, recent_tokens, boost, pad_nan)
        q[b, g * G:(g + 1) * G] = qg
        k[b, g] = kk
        v[b, g] = vv

    units = [(b, g) for b in range(B) for g in range(Hkv)]
    nthr = threads or default_threads()
    if nthr > 1 and len(units) > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(unit, units))
    else:
        for u_ in units:
            unit(u_)
    return DecodeInputs(q, k, v, seq, dtype)


def ragged_lengths(cfg: int, B: int, L: int, lo: int = 1, layer: int = 0) -> np.ndarray:
    """Seeded ragged sequence lengths in [lo, L] (the last row is always L)."""
    r = rng_for(cfg, T_LEN, layer)
    s = r.integers(lo, L + 1, size=B).astype(np.int32)
    if B:
        s[-1] = L
    return s


def poison_blocks(inp: DecodeInputs, keep) -> None:
    """Overwrite K and V of every block not in keep[b][g] with NaN (in place)."""
    B, _, Hkv, _, L = inp.shape
    nan = BF16_NAN if inp.dtype == "bf16" else np.float32(np.nan)
    nblk = -(-L // BLOCK)
    for b in range(B):
        for g in range(Hkv):
            ks = set(int(j) for j in keep[b][g])
            for j in range(nblk):
                if j not in ks:
                    inp.k[b, g, j * BLOCK:(j + 1) * BLOCK] = nan
                    inp.v[b, g, j * BLOCK:(j + 1) * BLOCK] = nan


def route_mask(n_layers: int = 36, n_full: int = 18, cfg: int = 5) -> np.ndarray:
    """Seeded per-layer hard route mask: 1 = full attention, 0 = sink+window."""
    perm = rng_for(cfg, T_ROUTE).permutation(n_layers)
    m = np.zeros(n_layers, dtype=np.uint8)
    m[perm[:n_full]] = 1
    return m


# Workload shapes (decode step of one attention layer unless noted).
WORKLOADS = {
    1: dict(name="tiny fp32 single-head 4K", B=1, Hq=1, Hkv=1, d=64, L=4096, dtype="f32",
            kind="gauss", topk=8, n_sink=1, n_recent=0),
    2: dict(name="llama3.1-8b dense decode 32K b8", B=8, Hq=32, Hkv=8, d=128, L=32768,
            dtype="bf16", kind="needles", splits=16),
    3: dict(name="centroid-sparse decode 128K b8", B=8, Hq=32, Hkv=8, d=128, L=131072,
            dtype="bf16", kind="mixture", topk=205, n_sink=1, n_recent=64, group=16, k_coarse=32,
            win_recent=128, tau=1e-3, phi=1e-4, patience=2, probe_dim=8, redraws="decode128k_b8"),
    4: dict(name="ART decode 64K b32", B=32, Hq=32, Hkv=8, d=128, L=65536, dtype="bf16",
            kind="recency", tau=1e-3, phi=1e-4, patience=2, probe_dim=8, redraws="art64k_b32"),
    5: dict(name="qwen3-8b 36-layer routed hybrid 256K b1", B=1, Hq=32, Hkv=8, d=128,
            L=262144, dtype="bf16", kind="needles", n_layers=36, n_full=18, n_shards=8,
            splits_per_shard=4, sa_splits=32, n_sink=1, n_recent=128),
}


# Units redrawn from later sub-seeds so that every decision of the full-size
# workloads clears the margins (top-k boundary gaps above 1e-4, every ART
# decision 1% away from the thresholds).  The table is data: it is written by
# tests/golden/make_redraws.py and read here, so the benchmark and the tests
# draw the same inputs.
REDRAWS_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                            "redraws.json")


def redraws(name: str) -> dict:
    """{(b, kvh): attempt} for a named workload (empty when the table has none)."""
    import json

    try:
        with open(REDRAWS_FILE) as f:
            table = json.load(f)
    except FileNotFoundError:
        return {}
    ent = table.get(name, {}).get("attempts", {})
    return {tuple(int(x) for x in key.split(",")): int(a) for key, a in ent.items()}


def workload_inputs(cfg: int, threads: int | None = None, **kw) -> DecodeInputs:
    """The full-size inputs of workload cfg, with its redrawn units applied."""
    W = WORKLOADS[cfg]
    attempts = redraws(W["redraws"]) if "redraws" in W else {}
    return make_inputs(cfg, W["B"], W["Hq"], W["Hkv"], W["d"], W["L"], dtype=W["dtype"], kind=W["kind"],
                       attempts=attempts, threads=threads, **kw)
