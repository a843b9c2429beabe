"""W8A8 FP8 projection (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

robotworld.top SparkDiffusion write-up, section 2.3: the attention linear
projections and the feed-forward layers run W8A8 in FP8 E4M3; weights carry a
static scale per output channel, calibrated offline, and activations a
dynamic scale per token computed at run time.

Readings where the page is silent:
  * a projection y = x W^T with W [N, K] (one row per output channel) is
    computed from the two quantised operands as
        y[m, n] = s_x[m] * s_w[n] * sum_k E4M3(xq[m, k]) * E4M3(wq[n, k]),
    i.e. the product of the dequantised operands; the oracle evaluates it in
    float64 (every term is an exact product of two E4M3 values);
  * the static weight quantisation is the per-row rule of the activation
    quantiser applied to W's rows: s_w[n] = max_k |W[n, k]| / 448, codes
    E4M3(W[n, k] * 448 / max_k |W[n, k]|), computed once, offline.
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode, quant_fp8_per_token


def quant_weight_per_channel(w_bits):
    """W [N, K] bf16 bits -> (codes uint8 [N, K], scales float32 [N]): the
    per-row activation rule applied to the weight's rows (one scale per
    output channel)."""
    return quant_fp8_per_token(w_bits)


def w8a8_gemm(xq, sx, wq, sw) -> np.ndarray:
    """y [M, N] float64 = diag(s_x) (E4M3(xq) E4M3(wq)^T) diag(s_w)."""
    X = e4m3_decode(np.asarray(xq))
    W = e4m3_decode(np.asarray(wq))
    acc = X @ W.T
    return acc * np.asarray(sx, dtype=np.float64)[:, None] * np.asarray(sw, dtype=np.float64)[None, :]


def w8a8_abs_products(xq, sx, wq, sw) -> np.ndarray:
    """sum_k |terms| of each output (scaled), the size an accumulation
    rounding error is proportional to."""
    X = np.abs(e4m3_decode(np.asarray(xq)))
    W = np.abs(e4m3_decode(np.asarray(wq)))
    return (X @ W.T) * np.abs(np.asarray(sx, dtype=np.float64))[:, None] * np.abs(
        np.asarray(sw, dtype=np.float64))[None, :]
