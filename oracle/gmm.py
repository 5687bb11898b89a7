"""Grouped matmul over expert bands in float64 (test infrastructure; see the
package docstring).

"Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e can't
hold": for every expert band of rows, the bf16 activations of the band are
multiplied by that expert's decoded and block-scaled weight; an expert with an
empty band produces no rows.  This oracle writes that definition out directly:
decode one expert's weight to float64, then one float64 matmul per band.  No
tiling, no fusion.

Activations arrive as bf16 bit patterns (uint16).  For the gate/up matmul the
band rows gather token rows through row_index (the sorted token of each row);
for the down matmul the input is already in band order (row_index None).
"""

import numpy as np

from .formats import decode_mxfp4, decode_nvfp4, e2m1_decode, e8m0_decode, e4m3_decode


def bf16_bits_to_f64(bits):
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dense_weights(w, e):
    """Dense float64 weight of expert e, laid out [N, K].

    w is a dict with 'fmt' ('mxfp4', 'nvfp4' or 'bf16'): 'codes' [E,N,K/2] and
    either 'scales' [E,N,K/32] (E8M0) or 'block_scales' [E,N,K/16] (E4M3) plus
    'tensor_scale' [E]; or, for the bf16 comparison arm of "Grouped matmul
    performance vs bf16", 'weights' [E,N,K] bf16 bit patterns."""
    if w["fmt"] == "mxfp4":
        return decode_mxfp4(w["codes"][e], w["scales"][e])
    if w["fmt"] == "nvfp4":
        return decode_nvfp4(w["codes"][e][None], w["block_scales"][e][None],
                            np.asarray(w["tensor_scale"])[e:e + 1])[0]
    if w["fmt"] == "bf16":
        return bf16_bits_to_f64(w["weights"][e])
    raise ValueError("unknown weight format %r" % (w["fmt"],))


def weight_columns(w):
    """N of the weight dict w."""
    return (w["weights"] if w["fmt"] == "bf16" else w["codes"]).shape[1]


def gmm(x_bits, row_index, group_offsets, w):
    """Y[r, :] = X[src(r), :] @ W[e]^T for every row r of band e, float64.

    x_bits: bf16 bits, [T, K] when row_index is given, else [M, K] in band order.
    row_index: [M] source row of each band row, or None for identity.
    group_offsets: [E+1] band boundaries.  Rows past group_offsets[E] are NaN
    (they belong to no band and are never written by the kernel).
    Returns Y [M, N] float64, M = len(row_index) or x rows."""
    return gmm_dense_x(bf16_bits_to_f64(x_bits), row_index, group_offsets, w)


def gmm_w4a4(xq_codes, xq_scales, row_index, group_offsets, w):
    """The W4A4 variant: the activations are given MXFP4-quantized (codes
    [rows, K/2], E8M0 scales [rows, K/32], see quant.py) and enter the same
    grouped matmul with their dequantized values."""
    from .formats import decode_mxfp4
    return gmm_dense_x(decode_mxfp4(xq_codes, xq_scales), row_index, group_offsets, w)


def gmm_dense_x(x, row_index, group_offsets, w):
    """gmm() on float64 activation rows x."""
    off = np.asarray(group_offsets, dtype=np.int64)
    E = off.size - 1
    M = len(row_index) if row_index is not None else x.shape[0]
    N = weight_columns(w)
    y = np.full((M, N), np.nan)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.arange(lo, hi)
        src = np.asarray(row_index, dtype=np.int64)[rows] if row_index is not None else rows
        W = dense_weights(w, e)                      # [N, K]
        y[lo:hi] = x[src] @ W.T
    return y


def _weight_column(w, e, n):
    """Decoded float64 column n of expert e's weight, length K."""
    if w["fmt"] == "bf16":
        return bf16_bits_to_f64(w["weights"][e, n])
    if w["fmt"] == "mxfp4":
        codes = w["codes"][e, n]
        v = e2m1_decode(np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(-1))
        return v * np.repeat(e8m0_decode(w["scales"][e, n]), 32)
    codes = w["codes"][e, n]
    v = e2m1_decode(np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(-1))
    return (v * np.repeat(e4m3_decode(w["block_scales"][e, n]), 16)
            * float(np.asarray(w["tensor_scale"])[e]))


def gmm_sampled(x_bits, row_index, group_offsets, w, rows, cols):
    """Y[rows[i], cols[i]] for sampled output positions, one dot product each.

    Same definition as gmm(), but decodes only the weight columns it needs so
    that full-size problems can be spot-checked.  A row outside every band
    gives NaN."""
    off = np.asarray(group_offsets, dtype=np.int64)
    out = np.empty(len(rows))
    for i, (r, c) in enumerate(zip(rows, cols)):
        r = int(r)
        if r >= off[-1]:
            out[i] = np.nan
            continue
        e = int(np.searchsorted(off, r, side="right") - 1)
        src = int(row_index[r]) if row_index is not None else r
        xr = bf16_bits_to_f64(x_bits[src])
        out[i] = float(np.dot(xr, _weight_column(w, e, int(c))))
    return out
