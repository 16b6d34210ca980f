"""Pure-Python brute force for tiny inputs (lists and math only, no numpy).

Used to pin the numpy oracle: every function here is written from the
textbook definition of softmax attention with explicit loops, independent of
the oracle's vectorised code.
"""

import math


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def softmax_attention(q, keys, values, scale):
    """Softmax(scale * <q, k_t>) weighted mean of the value rows (lists)."""
    if not keys:
        return [0.0] * len(q)
    logits = [scale * dot(q, k) for k in keys]
    top = max(logits)
    w = [math.exp(x - top) for x in logits]
    z = sum(w)
    return [sum(w[t] * values[t][i] for t in range(len(keys))) / z for i in range(len(values[0]))]


def attention_over_tokens(q, K, V, tokens, scale):
    return softmax_attention(q, [list(K[t]) for t in tokens], [list(V[t]) for t in tokens], scale)


def mean_rows(rows):
    n = len(rows)
    return [sum(r[i] for r in rows) / n for i in range(len(rows[0]))]
