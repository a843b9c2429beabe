"""Pins of the selector and causal-window oracle (oracle/variants.py).

robotworld.top SparkDiffusion write-up, section 2.1 (a fixed spatio-temporal
pattern as the selector of A_M) and section 4 (compensated sparse attention
restricted to a causal window for autoregressive video diffusion). Each
test ties one step to PyTorch's masked attention on the CPU in float64, a
closed form, a recurrence, brute force or an invariant.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import variants as ov
from workloads import synthetic


# --- causal window mask ---------------------------------------------------

def test_mask_closed_form_counts():
    for L, ct, W in [(60, 10, 0), (60, 10, 1), (60, 10, 2), (57, 8, 3), (16, 1, 0)]:
        M = ov.causal_window_mask(L, ct, W)
        for i in range(L):
            c = i // ct
            first = 0 if W == 0 else max(0, c - W + 1)
            lo, hi = first * ct, min(L, (c + 1) * ct)
            expect = np.zeros(L, dtype=bool)
            expect[lo:hi] = True
            assert (M[i] == expect).all(), (L, ct, W, i)


def test_mask_special_cases():
    assert (ov.causal_window_mask(32, 1, 0) == np.tril(np.ones((32, 32), dtype=bool))).all()
    assert ov.causal_window_mask(40, 40, 0).all()
    assert ov.causal_window_mask(40, 64, 1).all()
    M = ov.causal_window_mask(40, 8, 1)  # block diagonal
    blocks = np.kron(np.eye(5, dtype=int), np.ones((8, 8), dtype=int)).astype(bool)
    assert (M == blocks).all()


def test_block_allowed_interval_rule():
    # closed form: the query chunks of block b are [cq0, cq1], the key chunks
    # of block c are [ck0, ck1]; some pair is visible iff ck0 <= cq1 and
    # ck1 >= cq0 - W + 1 (W = 0: no lower limit)
    rng = np.random.default_rng(3)
    for _ in range(40):
        L = int(rng.integers(20, 300))
        bq = int(rng.choice([4, 8, 16]))
        bk = int(rng.choice([4, 8]))
        ct = int(rng.integers(1, 80))
        W = int(rng.integers(0, 4))
        A = ov.block_allowed(ov.causal_window_mask(L, ct, W), bq, bk)
        for b in range(A.shape[0]):
            cq0, cq1 = (b * bq) // ct, (min(L, (b + 1) * bq) - 1) // ct
            for c in range(A.shape[1]):
                ck0, ck1 = (c * bk) // ct, (min(L, (c + 1) * bk) - 1) // ct
                ok = ck0 <= cq1 and (W == 0 or ck1 >= cq0 - W + 1)
                assert A[b, c] == ok


# --- top-k among the allowed blocks ----------------------------------------

def test_topk_allowed_brute_force_rank():
    # a column is kept iff fewer than k allowed columns beat it (a higher
    # score, or an equal score at a lower index); padding counts the rest
    rng = np.random.default_rng(5)
    for _ in range(30):
        n_rows, n_cols = 6, int(rng.integers(1, 20))
        S = rng.integers(-3, 4, size=(n_rows, n_cols)).astype(np.float64)  # many ties
        allowed = rng.random((n_rows, n_cols)) < 0.6
        k = int(rng.integers(1, n_cols + 1))
        idx = ov.topk_block_map_allowed(S, k, allowed)
        for b in range(n_rows):
            cols = [c for c in range(n_cols) if allowed[b, c]]
            kept = sorted(c for c in cols
                          if sum(1 for o in cols if S[b, o] > S[b, c] or (S[b, o] == S[b, c] and o < c)) < k)
            n = len(kept)
            assert list(idx[b, :n]) == kept
            assert (idx[b, n:] == -1).all()


def test_topk_allowed_everything_is_plain_topk():
    rng = np.random.default_rng(6)
    S = rng.standard_normal((9, 30))
    for k in (1, 5, 30):
        assert (ov.topk_block_map_allowed(S, k, np.ones_like(S, dtype=bool)) == oracle.topk_block_map(S, k)).all()


# --- fixed spatio-temporal selector ------------------------------------------

def test_centroids_closed_form():
    T, Hg, Wg = 3, 5, 7
    L = T * Hg * Wg
    for bs in (4, 16, 64):
        cen = ov.block_centroids(L, bs, T, Hg, Wg)
        for b, (s, e) in enumerate(oracle.block_ranges(L, bs)):
            toks = range(s, e)
            expect = [sum(i // (Hg * Wg) for i in toks) / (e - s), sum((i // Wg) % Hg for i in toks) / (e - s),
                      sum(i % Wg for i in toks) / (e - s)]
            assert list(cen[b]) == expect


def test_fixed_scores_rows_as_blocks():
    # Wg = block size: each block is one (t, h) row, centroid (t, h, 31.5)
    T, Hg, Wg = 4, 5, 64
    L = T * Hg * Wg
    S = ov.fixed_block_scores(L, 64, 64, T, Hg, Wg)
    for b in range(T * Hg):
        for c in range(T * Hg):
            tb, hb, tc, hc = b // Hg, b % Hg, c // Hg, c % Hg
            assert S[b, c] == -float((tb - tc) ** 2 + (hb - hc) ** 2)
    allowed = np.ones_like(S, dtype=bool)
    idx = ov.topk_block_map_allowed(S, 1, allowed)
    assert (idx[:, 0] == np.arange(T * Hg)).all()  # itself, distance 0
    idx = ov.topk_block_map_allowed(S, 5, allowed)
    for t in range(1, T - 1):
        for h in range(1, Hg - 1):
            b = t * Hg + h
            assert sorted(idx[b]) == sorted([b, b - 1, b + 1, b - Hg, b + Hg])


def test_fixed_selector_one_dimensional_ties():
    # one row of 10 blocks of 64: block c is centred at 31.5 + 64 c; with
    # k = 2 the equidistant neighbours b-1 and b+1 tie and b-1 wins
    L = 640
    S = ov.fixed_block_scores(L, 64, 64, 1, 1, L)
    idx = ov.topk_block_map_allowed(S, 2, np.ones_like(S, dtype=bool))
    assert list(idx[0]) == [0, 1]
    for b in range(1, 10):
        assert list(idx[b]) == [b - 1, b]
    idx = ov.topk_block_map_allowed(S, 3, np.ones_like(S, dtype=bool))
    assert list(idx[4]) == [3, 4, 5] and list(idx[0]) == [0, 1, 2] and list(idx[9]) == [7, 8, 9]


# --- masked sparse branch ----------------------------------------------------

def _sdpa(Q, K, V, mask, scale):
    out = F.scaled_dot_product_attention(torch.tensor(Q)[None], torch.tensor(K)[None], torch.tensor(V)[None],
                                         attn_mask=torch.tensor(mask)[None], scale=scale)
    return out[0].numpy()


def test_sparse_masked_all_blocks_is_library_causal_attention():
    rng = np.random.default_rng(7)
    L, d = 200, 16
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    nk = math.ceil(L / 8)
    idx = np.tile(np.arange(nk), (math.ceil(L / 16), 1))
    for ct, W in [(1, 0), (24, 0), (24, 2), (50, 1)]:
        M = ov.causal_window_mask(L, ct, W)
        Os, r = ov.sparse_attention_masked(Q, K, V, idx, 16, 8, 0.3, M)
        ref = _sdpa(Q, K, V, M, 0.3)
        assert np.allclose(Os, ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(r, np.sqrt((ref * ref).mean(axis=1)), rtol=1e-12)
    # token-causal with chunk 1 is the textbook lower-triangular softmax
    Os, _ = ov.sparse_attention_masked(Q, K, V, idx, 16, 8, 0.3, ov.causal_window_mask(L, 1, 0))
    ref = F.scaled_dot_product_attention(torch.tensor(Q)[None], torch.tensor(K)[None], torch.tensor(V)[None],
                                         is_causal=True, scale=0.3)[0].numpy()
    assert np.allclose(Os, ref, rtol=1e-12, atol=1e-12)


def test_sparse_masked_kept_blocks_and_empty_rows():
    rng = np.random.default_rng(8)
    L, d, bq, bk = 96, 8, 16, 8
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    M = ov.causal_window_mask(L, 20, 1)
    idx = np.full((L // bq, 3), -1, dtype=np.int32)
    for b in range(L // bq):
        idx[b, :2] = [(2 * b) % (L // bk), (2 * b + 5) % (L // bk)]
    Os, r = ov.sparse_attention_masked(Q, K, V, idx, bq, bk, 0.5, M)
    keep = np.zeros((L, L), dtype=bool)
    for b in range(L // bq):
        for c in idx[b]:
            if c >= 0:
                keep[b * bq:(b + 1) * bq, c * bk:(c + 1) * bk] = True
    full = M & keep
    rows = full.any(axis=1)
    assert rows.sum() not in (0, L)  # the case has both kinds of row
    ref = _sdpa(Q, K, V, full, 0.5)
    assert np.allclose(Os[rows], ref[rows], rtol=1e-12, atol=1e-12)
    assert (Os[~rows] == 0).all() and (r[~rows] == 0).all()


def test_sparse_masked_without_mask_matches_unmasked_oracle():
    cfg = synthetic.TINY
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 0)
    f = oracle.bf16_bits_to_f64
    Q, K, V = f(Qb[0, :, 0]), f(Kb[0, :, 0]), f(Vb[0, :, 0])
    idx = oracle.topk_block_map(oracle.block_scores(Q, K, 64, 64), 4)
    a = ov.sparse_attention_masked(Q, K, V, idx, 64, 64, 0.125)
    b = oracle.sparse_attention(Q, K, V, idx, 64, 64, 0.125)
    assert np.allclose(a[0], b[0], rtol=1e-13, atol=1e-15) and np.allclose(a[1], b[1], rtol=1e-13)


# --- masked low-rank state ---------------------------------------------------

def test_lowrank_state_token_causal_recurrence():
    # chunk 1, no window: C_i = C_{i-1} + k~_i v_i^T (causal linear attention)
    rng = np.random.default_rng(9)
    L, r, d = 40, 4, 6
    kt, V = rng.standard_normal((L, r)), rng.standard_normal((L, d))
    C = ov.lowrank_states_masked(kt, V, ov.causal_window_mask(L, 1, 0), 1)
    run = np.zeros((r, d))
    for i in range(L):
        run = run + np.outer(kt[i], V[i])
        assert np.allclose(C[i], run, rtol=1e-13, atol=1e-13)


def test_lowrank_state_sliding_window_recurrence():
    # window W over chunks: C_c = C_{c-1} + X_c - X_{c-W}, X_c the chunk's own sum
    rng = np.random.default_rng(10)
    L, r, d, ct = 70, 3, 5, 9
    kt, V = rng.standard_normal((L, r)), rng.standard_normal((L, d))
    nch = math.ceil(L / ct)
    X = [kt[c * ct:(c + 1) * ct].T @ V[c * ct:(c + 1) * ct] for c in range(nch)]
    for W in (1, 2, 3):
        C = ov.lowrank_states_masked(kt, V, ov.causal_window_mask(L, ct, W), ct)
        run = np.zeros((r, d))
        for c in range(nch):
            run = run + X[c] - (X[c - W] if c - W >= 0 else 0)
            assert np.allclose(C[c], run, rtol=1e-12, atol=1e-12)


# --- the whole head ----------------------------------------------------------

def test_variant_head_reduces_to_plain_head():
    cfg = synthetic.TINY
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 0)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    g = synthetic.gen_gate(cfg)
    f = oracle.bf16_bits_to_f64
    Q, K, V = f(Qb[0, :, 1]), f(Kb[0, :, 1]), f(Vb[0, :, 1])
    kw = dict(T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q, bk=cfg.block_k, k_keep=4, sm_scale=0.125)
    a = oracle.rola_attention_head(Q, K, V, Q, K, f(Pqb), f(Pkb), g[0], **kw)
    b = ov.rola_attention_head_variant(Q, K, V, Q, K, f(Pqb), f(Pkb), g[0], **kw)
    assert (a["idx"] == b["idx"]).all()
    assert np.allclose(a["C"], b["C"][0], rtol=1e-13, atol=1e-13)
    assert np.allclose(a["O"], b["O"], rtol=1e-12, atol=1e-12)
    # a window that covers the whole sequence changes nothing either
    c = ov.rola_attention_head_variant(Q, K, V, Q, K, f(Pqb), f(Pkb), g[0], chunk_tokens=cfg.L, window=1, **kw)
    assert np.allclose(a["O"], c["O"], rtol=1e-12, atol=1e-12)


def test_variant_head_causal_blocks_never_look_ahead():
    cfg = synthetic.TINY
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 1)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    g = synthetic.gen_gate(cfg)
    f = oracle.bf16_bits_to_f64
    Q, K, V = f(Qb[0, :, 0]), f(Kb[0, :, 0]), f(Vb[0, :, 0])
    ct = cfg.Hg * cfg.Wg  # one latent frame per chunk
    for sel in ("topk", "fixed"):
        res = ov.rola_attention_head_variant(Q, K, V, Q, K, f(Pqb), f(Pkb), g[0], T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg,
                                             bq=64, bk=64, k_keep=4, sm_scale=0.125, select=sel,
                                             chunk_tokens=ct, window=2)
        for b, row in enumerate(res["idx"]):
            cq = (b * 64) // ct
            for c in row:
                if c >= 0:
                    assert cq - 2 < (c * 64) // ct <= cq
        # the first chunk's output depends on the first chunk only
        Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
        Q2[ct:] += 1.0
        K2[ct:] -= 0.5
        V2[ct:] *= 2.0
        res2 = ov.rola_attention_head_variant(Q2, K2, V2, Q2, K2, f(Pqb), f(Pkb), g[0], T=cfg.T, Hg=cfg.Hg,
                                              Wg=cfg.Wg, bq=64, bk=64, k_keep=4, sm_scale=0.125, select=sel,
                                              chunk_tokens=ct, window=2)
        if sel == "fixed":
            assert np.allclose(res["O"][:ct], res2["O"][:ct], rtol=1e-13, atol=1e-13)
        else:
            # the scored map of later query blocks moves, the first chunk's rows do not
            assert (res["idx"][: ct // 64] == res2["idx"][: ct // 64]).all()
            assert np.allclose(res["O"][:ct], res2["O"][:ct], rtol=1e-13, atol=1e-13)
