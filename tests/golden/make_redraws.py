"""Write tests/golden/redraws.json: the sub-seed of every full-size unit.

A (batch row, KV head) unit of a full-size workload is drawn from sub-seed
(attempt) 0 unless one of the method's decisions on it is too close to call:
then it is drawn again from sub-seed 1, 2, ... until every decision clears
its margin.  This is the input recipe's "score gaps > 1e-4" rule, decided by
the float64 oracle only (this script calls synth for the draws and oracle/
for the decisions, nothing else):

* top-k selection (Squeezed Attention blog, Q2 step 2): the gap between the
  k-th and (k+1)-th candidate score exceeds 1e-4; for two-level selection
  (Q2 step 4) the same holds at the coarse and at the fine boundary;
* ART (ART summary, §2.2-2.3): every stable step has d_scale < 0.99 tau and
  d_dir < 0.99 phi, every unstable one d_scale > 1.01 tau or d_dir > 1.01 phi,
  in each visit order the workload runs (block 0 then newest first; block 0
  then descending centroid score, §2.4; the top-k list, §2.4 over a
  selection).

Usage: python tests/golden/make_redraws.py [workload ...]  (about 5 minutes
on 8 cores).  The result is deterministic: for each unit the smallest passing
sub-seed.
"""

import json
import math
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle.art import art_margin_ok, importance_order  # noqa: E402
from oracle.selection import selection_gap, select_blocks, super_centroids, two_level_gaps  # noqa: E402

OUT = os.path.join(HERE, "redraws.json")
GAP = 1e-4
MAX_ATTEMPTS = 200

# workload name -> (synth cfg, decisions checked)
WORKLOADS = {"decode128k_b8": (3, ("topk", "two_level", "art_recency", "art_importance", "art_topk_list")),
             "art64k_b32": (4, ("art_recency",))}


def unit_ok(cfg, b, g, attempt, checks):
    """True when every listed decision of unit (b, g) drawn at `attempt` clears its margin."""
    W = synth.WORKLOADS[cfg]
    G, d, L = W["Hq"] // W["Hkv"], W["d"], W["L"]
    qg, k, v = synth.draw_unit(cfg, b, g, G, d, L, L, W["dtype"], W["kind"], attempt=attempt)
    up = lambda a: synth.bf16_to_f32(a).astype(np.float64)
    qf, kf, vf = up(qg)[None], up(k)[None, None], up(v)[None, None]
    del k, v
    seq = np.array([L], dtype=np.int32)
    scale = 1.0 / math.sqrt(d)
    nb = L // 64
    art = dict(tau=W["tau"], phi=W["phi"], patience=W["patience"], probe_dim=W["probe_dim"])

    def art_ok(order=None, n_visit=None):
        _, _, tr = oracle.art_decode(qf, kf, vf, seq, scale, order=order, n_visit=n_visit, **art)
        return all(art_margin_ok(t, W["tau"], W["phi"]) for t in tr.values())

    sig = None
    if {"topk", "two_level", "art_importance", "art_topk_list"} & set(checks):
        sig = oracle.centroid_scores(qf, oracle.block_centroids(kf, seq), seq, scale)[0, 0]
    for c in checks:
        if c == "topk" and not selection_gap(sig, nb, W["topk"], W["n_sink"], W["n_recent"]) > GAP:
            return False
        if c == "two_level":
            coarse = oracle.centroid_scores(qf, super_centroids(kf, seq, W["group"]), seq, scale,
                                            block=64 * W["group"])[0, 0]
            if not min(two_level_gaps(sig, coarse, nb, W["group"], W["k_coarse"], W["topk"], W["n_sink"],
                                      W["n_recent"])) > GAP:
                return False
        if c == "art_recency" and not art_ok():
            return False
        if c == "art_importance" and not art_ok(order=[[importance_order(sig.astype(np.float32), nb)]]):
            return False
        if c == "art_topk_list":
            lst = select_blocks(sig, nb, W["topk"], W["n_sink"], W["n_recent"])
            if not art_ok(order=[[lst + [0] * (nb - len(lst))]], n_visit=[[len(lst)]]):
                return False
    return True


def first_attempt(job):
    cfg, b, g, checks = job
    for a in range(MAX_ATTEMPTS):
        if unit_ok(cfg, b, g, a, checks):
            return (b, g), a
    raise RuntimeError(f"unit ({b},{g}) of cfg {cfg}: no passing sub-seed in {MAX_ATTEMPTS}")


def main(names):
    table = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            table = json.load(f)
    for name in names:
        cfg, checks = WORKLOADS[name]
        W = synth.WORKLOADS[cfg]
        t = time.time()
        jobs = [(cfg, b, g, checks) for b in range(W["B"]) for g in range(W["Hkv"])]
        with ProcessPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
            res = dict(ex.map(first_attempt, jobs))
        table[name] = {
            "workload": W["name"],
            "cfg": cfg,
            "checks": list(checks),
            "margins": "top-k gaps > 1e-4; every ART decision 1% clear of tau and phi",
            "written_by": "tests/golden/make_redraws.py",
            "attempts": {f"{b},{g}": a for (b, g), a in sorted(res.items()) if a},
        }
        print(f"{name}: {len(table[name]['attempts'])} of {len(jobs)} units redrawn, max attempt "
              f"{max(res.values())}, {time.time() - t:.0f}s", flush=True)
        with open(OUT, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or list(WORKLOADS))
