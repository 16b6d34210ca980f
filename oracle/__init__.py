"""Plain fp64 CPU oracle for block-sparse long-context decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the independent reference that the
HIP kernels are checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library itself never
does, and it imports nothing from the library.

Everything here is written for clarity, not speed: numpy in float64 on exact
upcasts of the bf16 / fp32 values the GPU sees, with one function per quantity
the method defines.  Sources (web pages, cited by title and section):

* "ART (Attention Run-time Termination)" technical summary (gist.science,
  paper 2606.00024): §2.1 streaming tile-wise accumulation, §2.2 the
  probe-based stop rule, §2.3 patience, §2.4 visit order, permutation
  invariance and the forced first block.
* "Squeezed Attention: Accelerating Long Context Length LLM Inference" Q&A
  blog (jaehun.me): Q1 worked example and Q2 steps 1-3 (centroids, comparing
  the query with centroids, attending to the selected keys only).
* "Pulsar Attention" technical summary (gist.science, paper 2607.20457):
  Phase 2, exact merge of per-shard attention by online softmax; Phase 1,
  the 64-token attention-sink prefix.
* "SparDA: Sparse Decoupled Attention" summary (gist.science, paper
  2606.04511): §2, one selector score per GQA group, no softmax in selection.
* "Flux Attention: Context-Aware Hybrid Attention" summary (gist.science,
  paper 2604.07394): §2, per-layer hard routing between full and sparse
  attention, decided once at prefill.

Parity status per function (what pins each one) is listed in the module
docstrings; every function here is pinned by at least one test in
``tests/test_oracle_*.py`` except where a docstring says "parity unpinned".
"""

from .attention import (
    EMPTY_STATE,
    block_ranges,
    split_ranges,
    head_state,
    merge_states,
    decode_dense,
    decode_split_states,
    decode_blocks,
    decode_sparse_split_states,
)
from .selection import block_centroids, centroid_scores, select_blocks, select_all
from .art import probe_metrics, art_decode_head, art_decode, default_order, importance_order
from .routing import routed_layer_outputs

__all__ = [
    "EMPTY_STATE",
    "block_ranges",
    "split_ranges",
    "head_state",
    "merge_states",
    "decode_dense",
    "decode_split_states",
    "decode_blocks",
    "decode_sparse_split_states",
    "block_centroids",
    "centroid_scores",
    "select_blocks",
    "select_all",
    "probe_metrics",
    "art_decode_head",
    "art_decode",
    "default_order",
    "importance_order",
    "routed_layer_outputs",
]
