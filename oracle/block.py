"""The steps either side of the attention in the deployment block (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

robotworld.top SparkDiffusion write-up, section 2.1: the low-rank branch
reuses the normalised q/k from before the backbone attention (q_norm),
and the backbone's own 3D RoPE is applied to q/k for the softmax branch;
the kais-engine portability report, section 2.1, lists the fused QKV +
RoPE operator and the scalar gate g = gate_proj(x) + gate_bias.

Readings where the pages are silent:
  * q/k RMSNorm normalises each token's whole projection row (all H*d
    channels) with a per-channel weight gamma and eps = 1e-6:
        y_c = x_c / sqrt(mean_c' x_c'^2 + eps) * gamma_c;
  * the backbone 3D RoPE on each head's d channels follows the same rule
    as the rank-truncated one of the low-rank branch, applied at full d:
    the split (d - 2 floor(d/3), floor(d/3), floor(d/3)) over (t, h, w),
    adjacent pairs inside each axis block, theta_m = 10000^(-2m/n_axis)
    (44/42/42 channels at d = 128);
  * the softmax branch takes Q = R(p) y, the low-rank branch the
    unrotated y (Qn); each is rounded to bfloat16 once, from the exact
    value (the oracle returns the exact float64 values);
  * the gate is one scalar per token, g_i = w . x_i + b, from the block's
    input row x_i (the activation that the FP8 quantiser also reads).
"""
from __future__ import annotations

import numpy as np

from .attention import rope_pairs, rope_rotate


def rms_norm_rows(X: np.ndarray, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gamma per row of X [L, C] (float64)."""
    X = np.asarray(X, dtype=np.float64)
    y = X / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    return y


def qk_norm_rope(X: np.ndarray, H: int, d: int, pos: np.ndarray, gamma=None, eps: float = 1e-6):
    """Fused q (or k) producer: X [L, H*d] -> (Xn, Xr), both [L, H, d] float64.

    Xn = RMSNorm(X) (pre-RoPE, for the low-rank branch); Xr = the backbone
    3D RoPE at positions pos [L, 3] applied to every head of Xn.
    """
    Y = rms_norm_rows(X, gamma, eps)
    L = Y.shape[0]
    Xn = Y.reshape(L, H, d)
    pairs = rope_pairs(d)
    Xr = np.stack([rope_rotate(Xn[:, h, :], pos, pairs) for h in range(H)], axis=1)
    return Xn, Xr


def gate_gemv(X: np.ndarray, w, b: float) -> np.ndarray:
    """g_i = w . x_i + b for X [L, C] (float64)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(w, dtype=np.float64) + float(b)


def gate_abs_terms(X: np.ndarray, w) -> np.ndarray:
    """sum_c |w_c x_ic| per row, the size a summation error is proportional to."""
    return np.abs(np.asarray(X, dtype=np.float64)) @ np.abs(np.asarray(w, dtype=np.float64))
