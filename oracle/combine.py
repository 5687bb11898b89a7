"""Top-k weighted unpermute (test infrastructure; see the package docstring).

Each token's output is the router-weighted sum of the rows its k pairs were
sorted to.  The pages do not write the formula out; it follows from the band
layout ("Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e
can't hold") and from the rule that the expert reduction is deterministic,
summing in a fixed order without atomics ("DeepSeek-V4-Flash" PocketLLM docs,
section "Correctness and precision").  Slots are summed in ascending j, in
float64.  A dropped pair (pair_row -1) contributes nothing.
"""

import numpy as np


def combine(y, topk_weights, pair_row):
    """out[t, :] = sum_j topk_weights[t, j] * y[pair_row[t*k + j], :], float64."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = w.shape
    pr = np.asarray(pair_row, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, y.shape[1]))
    for j in range(k):
        r = pr[:, j]
        ok = r >= 0
        out[ok] += w[ok, j, None] * y[r[ok]]
    return out
