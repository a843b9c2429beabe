"""Pins of the deployment-block producer steps of the oracle (q/k RMSNorm +
backbone 3D RoPE, the scalar gate) against a library routine, brute force,
closed forms and invariants (robotworld.top SparkDiffusion write-up, section
2.1: normalised q/k reused by the low-rank branch; kais-engine report,
section 2.1: fused QKV + RoPE operator and the scalar gate)."""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def test_rms_norm_matches_library():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((40, 5120)) * rng.uniform(0.1, 10, size=(40, 1))
    gamma = 1 + 0.1 * rng.standard_normal(5120)
    ref = F.rms_norm(torch.tensor(X), (5120,), weight=torch.tensor(gamma), eps=1e-6).numpy()
    assert np.allclose(oracle.rms_norm_rows(X, gamma, 1e-6), ref, rtol=1e-13, atol=1e-15)


def test_rms_norm_closed_form():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((10, 256)) * 1e-3   # small rows: eps matters
    eps = 1e-6
    Y = oracle.rms_norm_rows(X, None, eps)
    m = (X * X).mean(axis=1)
    assert np.allclose((Y * Y).mean(axis=1), m / (m + eps), rtol=1e-13)
    assert np.array_equal(np.sign(Y), np.sign(X))
    # scale invariance up to eps
    assert np.allclose(oracle.rms_norm_rows(1e3 * X, None, 0.0), oracle.rms_norm_rows(X, None, 0.0), rtol=1e-13)


def test_backbone_rope_split_at_full_head_dim():
    pairs = oracle.rope_pairs(128)
    axes = [a for _, a, _ in pairs]
    # 44/42/42 channels over (t, h, w): 22 + 21 + 21 pairs, every channel rotated
    assert axes == [0] * 22 + [1] * 21 + [2] * 21
    dims = [dm for dm, _, _ in pairs]
    assert dims == list(range(0, 128, 2))
    assert pairs[22][2] == 1.0 and pairs[43][2] == 1.0
    assert math.isclose(pairs[23][2], 10000 ** (-2 / 42), rel_tol=1e-15)


def test_qk_norm_rope_brute_force_tiny():
    # two heads of d = 8 (pairs (0,1),(2,3) on t, (4,5) on h, (6,7) on w), each
    # head rotated pair by pair as complex multiplication, by hand
    rng = np.random.default_rng(2)
    H, d, L = 2, 8, 5
    X = rng.standard_normal((L, H * d))
    pos = rng.integers(0, 9, size=(L, 3))
    gamma = rng.uniform(0.5, 1.5, size=H * d)
    Xn, Xr = oracle.qk_norm_rope(X, H, d, pos, gamma, 1e-6)
    for i in range(L):
        ms = sum(v * v for v in X[i]) / (H * d)
        y = [X[i, c] / math.sqrt(ms + 1e-6) * gamma[c] for c in range(H * d)]
        for h in range(H):
            for c in range(d):
                assert math.isclose(Xn[i, h, c], y[h * d + c], rel_tol=1e-13)
            # split of d = 8: t gets 8 - 2*2 = 4 dims (2 pairs), h and w 2 each
            for dim, axis, theta in [(0, 0, 1.0), (2, 0, 10000 ** (-2 / 4)), (4, 1, 1.0), (6, 2, 1.0)]:
                z = complex(y[h * d + dim], y[h * d + dim + 1]) * complex(math.cos(pos[i, axis] * theta),
                                                                          math.sin(pos[i, axis] * theta))
                assert math.isclose(Xr[i, h, dim], z.real, rel_tol=1e-12, abs_tol=1e-14)
                assert math.isclose(Xr[i, h, dim + 1], z.imag, rel_tol=1e-12, abs_tol=1e-14)


def test_backbone_rope_relative_position_and_norm():
    # per head: |R(p) y| = |y|, R(0) = I, and (R(p) a) . (R(p') b) depends on p - p' only
    rng = np.random.default_rng(3)
    H, d, L = 3, 128, 30
    X = rng.standard_normal((L, H * d))
    pos = rng.integers(0, 60, size=(L, 3))
    Xn, Xr = oracle.qk_norm_rope(X, H, d, pos)
    assert np.allclose(np.linalg.norm(Xr, axis=2), np.linalg.norm(Xn, axis=2), rtol=1e-13)
    _, X0 = oracle.qk_norm_rope(X, H, d, np.zeros_like(pos))
    assert np.array_equal(X0, Xn)
    shift = rng.integers(-20, 20, size=(1, 3))
    _, Xs = oracle.qk_norm_rope(X, H, d, pos + shift)
    for h in range(H):
        assert np.allclose(Xr[:, h] @ Xr[:, h].T, Xs[:, h] @ Xs[:, h].T, rtol=1e-11, atol=1e-11)


def test_gate_brute_force_and_bound_terms():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 50))
    w = rng.standard_normal(50) * 0.1
    g = oracle.gate_gemv(X, w, 0.05)
    for i in range(6):
        assert math.isclose(g[i], sum(w[c] * X[i, c] for c in range(50)) + 0.05, rel_tol=1e-13)
    t = oracle.gate_abs_terms(X, w)
    assert (t >= np.abs(g - 0.05) - 1e-15).all()
    assert math.isclose(t[0], sum(abs(w[c] * X[0, c]) for c in range(50)), rel_tol=1e-13)
