"""Gate/up activation after the fused w13 matmul (test infrastructure; see the
package docstring).

"Running DeepSeek V4 Flash on TPU v6", section "Grouped matmul performance vs
bf16", names the gate/up activation that follows w13 (the fused gate+up
matmul; the "DeepSeek-V4-Flash-0731-NVFP4" model card, section "The lossless
weight cast", calls it the fused w1/w3 GEMM1) but does not write it out.  The
reading taken here is the SiLU-gated product of the two halves of w13's
output: the first N/2 columns are the gate (w1), the last N/2 the up
projection (w3), and

    h[r, j] = silu(y[r, j]) * y[r, N/2 + j],   silu(z) = z / (1 + exp(-z)),

computed in float64.
"""

import numpy as np


def silu(z):
    """z * sigmoid(z) in float64; exp(-z) overflowing to inf gives -0."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_mul(y):
    """[M, N] w13 output -> [M, N/2] activation: silu(gate) * up."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[1]
    if n % 2:
        raise ValueError("the fused gate/up output needs an even column count")
    h = n // 2
    return silu(y[:, :h]) * y[:, h:]
