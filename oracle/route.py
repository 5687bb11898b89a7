"""Expert-sorted token layout (test infrastructure; see the package docstring).

Source: "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e
can't hold".  This module turns the router's top-k choices into the layout
the grouped matmul consumes: every (token, slot) pair becomes one row, rows
are grouped by the expert they go to, and group_offsets gives where each
expert's rows start and end.  The page leaves the order of rows within one
expert open; here they keep increasing flat pair index p = t * k + j (a stable
sort), which makes every index array unique and comparable bit for bit.

A pair whose expert id lies outside [0, E) belongs to no band: it is dropped,
counted, and its pair_row is -1.
"""

import numpy as np


def route_sort(topk_ids, E):
    """Counting sort of token-expert pairs into expert bands.

    topk_ids: [T, k] integer expert ids (slot j of token t is pair p = t*k + j).
    Returns a dict of int32 arrays:
      group_offsets [E+1]  band e is rows [group_offsets[e], group_offsets[e+1])
      sorted_token  [T*k]  token of each band row (rows past the last band: -1)
      sorted_pair   [T*k]  pair index of each band row (likewise -1)
      pair_row      [T*k]  band row of each pair (-1 for dropped pairs)
      err_count     int    number of dropped pairs
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    M = T * k
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    # Stable order of the valid pairs by expert id (ties keep pair order).
    valid_pairs = np.nonzero(valid)[0]
    order = valid_pairs[np.argsort(flat[valid_pairs], kind="stable")]
    n_valid = order.size
    sorted_pair = np.full(M, -1, dtype=np.int64)
    sorted_pair[:n_valid] = order
    sorted_token = np.full(M, -1, dtype=np.int64)
    sorted_token[:n_valid] = order // k
    pair_row = np.full(M, -1, dtype=np.int64)
    pair_row[order] = np.arange(n_valid)
    return {
        "group_offsets": offsets.astype(np.int32),
        "sorted_token": sorted_token.astype(np.int32),
        "sorted_pair": sorted_pair.astype(np.int32),
        "pair_row": pair_row.astype(np.int32),
        "err_count": int(M - n_valid),
    }
