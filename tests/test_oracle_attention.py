"""Pins of the attention oracle against things other than itself.

Each test ties one oracle step to a library routine (PyTorch's attention,
pooling and ELU on the CPU in float64), a hand-worked fixture, a closed
form, brute force or an invariant fixed by the method's statement
(robotworld.top SparkDiffusion write-up, section 2.1).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_head(seed=0, cfg=synthetic.TINY):
    Q, K, V = synthetic.gen_qkv(cfg, seed)
    f = oracle.bf16_bits_to_f64
    return cfg, f(Q[0, :, 0]), f(K[0, :, 0]), f(V[0, :, 0])


# --- block map ------------------------------------------------------------

def test_block_map_hand_worked_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "block_map_worked.json")))
    Q = np.array(fx["Q"], dtype=np.float64)
    K = np.array(fx["K"], dtype=np.float64)
    S = oracle.block_scores(Q, K, fx["block_q"], fx["block_k"])
    assert (S == np.array(fx["scores"])).all()
    assert (oracle.topk_block_map(S, fx["k_keep"]) == np.array(fx["expected_idx"])).all()
    tc = fx["tie_case"]
    assert (oracle.topk_block_map(S, tc["k_keep"]) == np.array(tc["expected_idx"])).all()


def test_pooled_means_match_library_avg_pool():
    rng = np.random.default_rng(1)
    for L, bs in [(256, 64), (250, 64), (1000, 128), (7, 4)]:
        X = rng.standard_normal((L, 8))
        ref = F.avg_pool1d(torch.tensor(X.T[None]), bs, bs, ceil_mode=True)[0].numpy().T
        assert np.allclose(oracle.pooled_means(X, bs), ref, rtol=1e-13, atol=1e-14)


def test_block_ranges_cover_and_tail():
    r = oracle.block_ranges(32760, 128)
    assert len(r) == 256 and r[-1] == (32640, 32760)
    r = oracle.block_ranges(75600, 64)
    assert len(r) == 1182 and r[-1][1] - r[-1][0] == 16
    r = oracle.block_ranges(75600, 128)
    assert len(r) == 591 and r[-1][1] - r[-1][0] == 80


def test_topk_constructed_known_answer():
    # key-block means c*e_c, query-block means the indicator of a chosen set:
    # S[b, c] = (c + 1) * [c in A_b], so the top-k set is A_b by construction.
    rng = np.random.default_rng(2)
    n_q, n_k, k = 6, 10, 3
    bq, bk = 4, 2
    sets = [np.sort(rng.choice(n_k, size=k, replace=False)) for _ in range(n_q)]
    Q = np.zeros((n_q * bq, n_k))
    K = np.zeros((n_k * bk, n_k))
    for c in range(n_k):
        K[c * bk:(c + 1) * bk, c] = c + 1.0
    for b, A in enumerate(sets):
        Q[b * bq:(b + 1) * bq, A] = 1.0
    S = oracle.block_scores(Q, K, bq, bk)
    got = oracle.topk_block_map(S, k)
    for b in range(n_q):
        assert list(got[b]) == list(sets[b])


def test_topk_brute_force_and_invariants():
    rng = np.random.default_rng(3)
    S = rng.integers(-3, 4, size=(40, 9)).astype(np.float64)  # many ties
    for k in (1, 4, 9):
        idx = oracle.topk_block_map(S, k)
        for b in range(S.shape[0]):
            row = idx[b]
            assert len(set(row)) == k and (np.diff(row) > 0).all()
            kept = set(row.tolist())
            # brute force: every kept block beats every dropped one under
            # (score descending, index ascending)
            for c in kept:
                for e in set(range(9)) - kept:
                    assert (S[b, c] > S[b, e]) or (S[b, c] == S[b, e] and c < e)
    assert (oracle.topk_block_map(S, 9) == np.arange(9)).all()


def test_keep_count_readme_ratios():
    # README_zh: keep ratio 0.1 / 0.05 / 0.03 <-> sparsity 90 / 95 / 97 %
    assert oracle.keep_count(0.75, 16) == 4
    assert oracle.keep_count(0.90, 512) == 52
    assert oracle.keep_count(0.95, 512) == 26
    assert oracle.keep_count(0.97, 1182) == 36
    assert oracle.keep_count(0.90, 1182) == 119
    assert oracle.keep_count(0.0, 100) == 100
    assert oracle.keep_count(0.999999, 100) == 1
    for s in (0.9, 0.95, 0.97):
        for n in (16, 100, 512, 1182):
            k = oracle.keep_count(s, n)
            assert k / n >= 1 - s - 1e-12 and (k - 1) / n < 1 - s


# --- sparse branch --------------------------------------------------------

def test_sparse_branch_full_keep_is_dense_attention():
    cfg, Q, K, V = _tiny_head()
    L = cfg.L
    n_k = L // cfg.block_k
    idx = np.tile(np.arange(n_k, dtype=np.int32), (L // cfg.block_q, 1))
    Os, r = oracle.sparse_attention(Q, K, V, idx, cfg.block_q, cfg.block_k, 1 / math.sqrt(cfg.d))
    ref = F.scaled_dot_product_attention(torch.tensor(Q)[None], torch.tensor(K)[None],
                                         torch.tensor(V)[None])[0].numpy()
    assert np.allclose(Os, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(r, np.sqrt((ref ** 2).mean(axis=1)), rtol=1e-12)


@pytest.mark.parametrize("L,bq,bk,k", [(1024, 64, 64, 4), (300, 128, 64, 2), (200, 64, 64, 1)])
def test_sparse_branch_matches_library_masked_attention(L, bq, bk, k):
    rng = np.random.default_rng(L)
    d = 32
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    S = oracle.block_scores(Q, K, bq, bk)
    idx = oracle.topk_block_map(S, k)
    Os, _ = oracle.sparse_attention(Q, K, V, idx, bq, bk, 0.3)
    # boolean mask built from the block map, handed to the library routine
    mask = np.zeros((L, L), dtype=bool)
    for b in range(idx.shape[0]):
        for c in idx[b]:
            mask[b * bq:(b + 1) * bq, c * bk:(c + 1) * bk] = True
    ref = F.scaled_dot_product_attention(torch.tensor(Q)[None], torch.tensor(K)[None], torch.tensor(V)[None],
                                         attn_mask=torch.tensor(mask)[None], scale=0.3)[0].numpy()
    assert np.allclose(Os, ref, rtol=1e-12, atol=1e-12)


# --- low-rank branch ------------------------------------------------------

def test_phi_is_elu_plus_one():
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(oracle.phi_elu1(x), F.elu(torch.tensor(x)).numpy() + 1.0, rtol=1e-15, atol=1e-15)
    assert (oracle.phi_elu1(x) > 0).all()


def test_positions_raster_order():
    pos = oracle.token_positions(3, 4, 5)
    assert tuple(pos[0]) == (0, 0, 0)
    assert tuple(pos[1]) == (0, 0, 1)
    assert tuple(pos[5]) == (0, 1, 0)
    assert tuple(pos[20]) == (1, 0, 0)
    assert tuple(pos[59]) == (2, 3, 4)


def test_rope_pairs_split():
    p16 = oracle.rope_pairs(16)
    # 6/5/5 dims over (t, h, w): pairs (0,1),(2,3),(4,5) | (6,7),(8,9) | (11,12),(13,14)
    assert [(d, a) for d, a, _ in p16] == [(0, 0), (2, 0), (4, 0), (6, 1), (8, 1), (11, 2), (13, 2)]
    p32 = oracle.rope_pairs(32)
    assert [d for d, _, _ in p32] == [0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 28, 30]
    assert [a for _, a, _ in p32] == [0] * 6 + [1] * 5 + [2] * 5
    # theta_0 = 1 on every axis; theta_m = 10000^(-2m/n) (n = 12 on t at r=32)
    assert p32[0][2] == 1.0 and p32[6][2] == 1.0 and p32[11][2] == 1.0
    assert math.isclose(p32[1][2], 10000 ** (-2 / 12), rel_tol=1e-15)


def test_rope_is_complex_rotation():
    # R(p) acts on each pair as multiplication by exp(i * p_axis * theta)
    rng = np.random.default_rng(4)
    a = rng.standard_normal((50, 32))
    pos = rng.integers(0, 80, size=(50, 3))
    pairs = oracle.rope_pairs(32)
    out = oracle.rope_rotate(a, pos, pairs)
    for dim, axis, theta in pairs:
        z = (a[:, dim] + 1j * a[:, dim + 1]) * np.exp(1j * pos[:, axis] * theta)
        assert np.allclose(out[:, dim], z.real, atol=1e-13) and np.allclose(out[:, dim + 1], z.imag, atol=1e-13)
    assert np.allclose(np.linalg.norm(out, axis=1), np.linalg.norm(a, axis=1), rtol=1e-13)
    assert np.array_equal(oracle.rope_rotate(a, np.zeros_like(pos), pairs), a)


@pytest.mark.parametrize("rank", [16, 32])
def test_rope_relative_position_invariance(rank):
    # q~_i . k~_j depends only on p_i - p_j (RoPE applied after phi keeps
    # relative spatio-temporal geometry, section 2.1)
    rng = np.random.default_rng(rank)
    d, n = 64, 40
    Pq = rng.standard_normal((rank, d)) / 8
    Pk = rng.standard_normal((rank, d)) / 8
    qn = rng.standard_normal((n, d))
    kn = rng.standard_normal((n, d))
    pos_q = rng.integers(0, 50, size=(n, 3))
    pos_k = rng.integers(0, 50, size=(n, 3))
    pairs = oracle.rope_pairs(rank)
    shift = rng.integers(-20, 20, size=(1, 3))
    dots = oracle.lowrank_features(qn, Pq, pos_q, pairs) @ oracle.lowrank_features(kn, Pk, pos_k, pairs).T
    dots2 = oracle.lowrank_features(qn, Pq, pos_q + shift, pairs) @ oracle.lowrank_features(kn, Pk, pos_k + shift, pairs).T
    assert np.allclose(dots, dots2, rtol=1e-12, atol=1e-12)
    # and it does depend on the relative position (the rotation is not a no-op)
    dots3 = oracle.lowrank_features(qn, Pq, pos_q + shift, pairs) @ oracle.lowrank_features(kn, Pk, pos_k, pairs).T
    assert not np.allclose(dots, dots3, atol=1e-6)


def test_lowrank_state_associativity_brute_force():
    # q~_i^T C == sum_j (q~_i . k~_j) v_j, one query at a time
    cfg, Q, K, V = _tiny_head(1)
    Pq, Pk = (oracle.bf16_bits_to_f64(p) for p in synthetic.gen_lowrank_params(cfg))
    pos = oracle.token_positions(cfg.T, cfg.Hg, cfg.Wg)
    pairs = oracle.rope_pairs(cfg.rank)
    qt = oracle.lowrank_features(Q, Pq, pos, pairs)
    kt = oracle.lowrank_features(K, Pk, pos, pairs)
    C = oracle.lowrank_state(kt, V)
    assert C.shape == (cfg.rank, cfg.d)
    for i in (0, 17, 500, cfg.L - 1):
        brute = np.zeros(cfg.d)
        for j in range(cfg.L):
            brute += float(qt[i] @ kt[j]) * V[j]
        assert np.allclose(qt[i] @ C, brute, rtol=1e-11, atol=1e-10)


def test_rmsnorm_closed_form_and_scale_invariance():
    rng = np.random.default_rng(6)
    qt = rng.standard_normal((30, 16))
    C = rng.standard_normal((16, 64))
    eps = 1e-6
    O = oracle.lowrank_output(qt, C, eps)
    y = qt @ C
    m = (y * y).mean(axis=1)
    assert np.allclose((O * O).mean(axis=1), m / (m + eps), rtol=1e-12)
    assert np.allclose(oracle.lowrank_output(qt, 1e3 * C, eps), O, rtol=1e-6)
    # sign: O_lr points along y
    assert (np.sign(O) == np.sign(y)).all()
    gamma = rng.uniform(0.5, 2, size=64)
    assert np.allclose(oracle.lowrank_output(qt, C, eps, gamma), O * gamma, rtol=1e-14)


# --- fusion and the whole layer -------------------------------------------

def _layer(gate, heads=None, cfg=synthetic.TINY):
    Q, K, V = synthetic.gen_qkv(cfg, 0)
    Pq, Pk = synthetic.gen_lowrank_params(cfg)
    k = oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))
    return oracle.rola_attention(Q, K, V, Pq, Pk, gate, T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg,
                                 bq=cfg.block_q, bk=cfg.block_k, k_keep=k, heads=heads)


def test_zero_gate_is_pure_sparse_branch():
    cfg = synthetic.TINY
    res = _layer(np.zeros((1, cfg.L)))
    for v in res.values():
        assert np.array_equal(v["O"], v["Os"])


def test_unit_gate_recomposition():
    cfg = synthetic.TINY
    g = np.ones((1, cfg.L))
    res = _layer(g, heads=[(0, 1)])
    v = res[(0, 1)]
    assert np.allclose(v["O"], v["Os"] + v["r"][:, None] * v["Olr"], rtol=1e-15, atol=1e-15)
    # the gate enters linearly
    g2 = 2.5 * g
    v2 = _layer(g2, heads=[(0, 1)])[(0, 1)]
    assert np.allclose(v2["O"] - v["Os"], 2.5 * (v["O"] - v["Os"]), rtol=1e-12, atol=1e-14)


def test_tiny_layer_shapes_and_keep_count():
    cfg = synthetic.TINY
    res = _layer(synthetic.gen_gate(cfg))
    v = res[(0, 0)]
    assert v["idx"].shape == (16, 4)
    assert v["O"].shape == (cfg.L, cfg.d) and v["C"].shape == (16, 64)
    assert np.isfinite(v["O"]).all()
