"""RoLA compensated sparse attention, step by step, in float64 (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring). Layout of Q, K, V and
of every per-token output: [B, L, H, d] with d contiguous; bf16 inputs come
in as uint16 bit patterns and are widened exactly to float64.

Method, robotworld.top SparkDiffusion write-up, section 2.1:
  A~ = A_M + g (.) C_psi: a block-sparse softmax branch A_M that keeps a
  1-s fraction of query/key blocks, plus a low-rank compensation branch
  q~_i = R_r(p_i) phi(P_q q_i), k~_j = R_r(p_j) phi(P_k k_j),
  C = sum_j k~_j v_j^T, O_lr,i = RMSNorm(q~_i^T C), fused per token as
  O_i = O_s,i + g_i r_i O_lr,i with r_i the RMS of O_s,i.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Block partition and block map (section 2.1: the sparse branch keeps a 1-s
# fraction of query-key blocks, chosen by top-k over block-level scores).
# ---------------------------------------------------------------------------

def block_ranges(L: int, bs: int):
    """Token ranges of consecutive blocks of size bs; the last may be partial.

    Reading: tokens are in raster order and blocks are consecutive runs of
    that order; a partial tail block holds only its valid tokens.
    """
    return [(s, min(L, s + bs)) for s in range(0, L, bs)]


def pooled_means(X: np.ndarray, bs: int) -> np.ndarray:
    """Mean of the tokens of each block: X [L, d] -> [n_blocks, d].

    Reading: a block is summarised by the plain mean of its valid tokens.
    """
    L = X.shape[0]
    return np.stack([X[s:e].sum(axis=0) / (e - s) for s, e in block_ranges(L, bs)])


def block_scores(Q: np.ndarray, K: np.ndarray, bq: int, bk: int) -> np.ndarray:
    """Block-level scores S[b, c] = mean(Q over block b) . mean(K over block c).

    Reading: the pages say only "block-level scoring"; the score is the raw
    dot product of the pooled means (a positive scale or a row softmax would
    leave the top-k set unchanged).
    """
    return pooled_means(Q, bq) @ pooled_means(K, bk).T


def keep_count(sparsity: float, n_kblocks: int) -> int:
    """Key blocks kept per query block for sparsity s.

    README_zh (single-sample inference): `topk` is the kept fraction, so
    0.1 / 0.05 / 0.03 mean 90 / 95 / 97% sparsity. Reading: round up, so
    the kept fraction is at least 1-s, with at least one and at most all.
    """
    k = math.ceil((1.0 - sparsity) * n_kblocks - 1e-9)
    return int(min(max(k, 1), n_kblocks))


def topk_block_map(S: np.ndarray, k: int) -> np.ndarray:
    """For each row of S the k largest columns, listed in ascending order.

    Reading: equal scores at the threshold go to the lower block index.
    """
    n_rows, n_cols = S.shape
    out = np.empty((n_rows, k), dtype=np.int32)
    cols = np.arange(n_cols)
    for b in range(n_rows):
        order = np.lexsort((cols, -S[b]))  # by score descending, then index
        out[b] = np.sort(order[:k])
    return out


# ---------------------------------------------------------------------------
# Sparse branch A_M (section 2.1).
# ---------------------------------------------------------------------------

def dense_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(Q K^T * sm_scale) V for one head; Q [Lq, d], K/V [Lk, d]."""
    logits = (Q @ K.T) * sm_scale
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ V


def sparse_attention(Q, K, V, idx, bq: int, bk: int, sm_scale: float):
    """Block-sparse softmax attention for one head.

    Q [Lq, d], K, V [L, d]; idx [Nq, k] kept key blocks per query block
    (Q may be a run of whole query blocks, with idx the matching rows). Each
    query of block b attends, with an ordinary softmax, to exactly the valid
    keys of the blocks idx[b]. Returns (O_s [Lq, d], r [Lq]) where r is the
    RMS of each output row over d (section 2.1: r_i is the RMS of O_s,i).
    Reading: r is per (token, head), over the head dimension.
    """
    L, d = Q.shape
    kr = block_ranges(K.shape[0], bk)
    Os = np.empty((L, d))
    for b, (s, e) in enumerate(block_ranges(L, bq)):
        keys = np.concatenate([np.arange(*kr[c]) for c in idx[b]])
        Os[s:e] = dense_attention(Q[s:e], K[keys], V[keys], sm_scale)
    r = np.sqrt(np.mean(Os * Os, axis=1))
    return Os, r


# ---------------------------------------------------------------------------
# Low-rank compensation branch C_psi (section 2.1).
# ---------------------------------------------------------------------------

def phi_elu1(x: np.ndarray) -> np.ndarray:
    """phi(x) = ELU(x) + 1: x + 1 for x > 0, exp(x) otherwise."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def token_positions(T: int, Hg: int, Wg: int) -> np.ndarray:
    """Raster positions p_i = (t, h, w) with i = (t*Hg + h)*Wg + w; [L, 3]."""
    pos = np.empty((T * Hg * Wg, 3), dtype=np.int64)
    i = 0
    for t in range(T):
        for h in range(Hg):
            for w in range(Wg):
                pos[i] = (t, h, w)
                i += 1
    return pos


def rope_pairs(rank: int, base: float = 10000.0):
    """The rotated pairs of the rank-truncated 3D RoPE: (dim, axis, theta).

    Section 2.1 names a rank-truncated 3D RoPE R_r(p) on the rank-r features
    without spelling it out. Reading: the r feature dims are split over the
    axes (t, h, w) as (r - 2*floor(r/3), floor(r/3), floor(r/3)) in that
    order (6/5/5 at r = 16); inside each axis block adjacent dims
    (2m, 2m+1) form a pair rotated by the angle p_axis * theta_m with
    theta_m = base^(-2m / n_axis); an odd last dim of a block is not rotated.
    """
    n = (rank - 2 * (rank // 3), rank // 3, rank // 3)
    pairs = []
    start = 0
    for axis, na in enumerate(n):
        for m in range(na // 2):
            pairs.append((start + 2 * m, axis, base ** (-2.0 * m / na)))
        start += na
    return pairs


def rope_rotate(a: np.ndarray, pos: np.ndarray, pairs) -> np.ndarray:
    """Apply R_r(p_i) to each row a_i of a [L, r]: rotate every pair
    (u, v) -> (u cos x - v sin x, u sin x + v cos x), x = p_i[axis] * theta.
    """
    out = a.copy()
    for dim, axis, theta in pairs:
        ang = pos[:, axis] * theta
        c, s = np.cos(ang), np.sin(ang)
        u, v = a[:, dim], a[:, dim + 1]
        out[:, dim] = u * c - v * s
        out[:, dim + 1] = u * s + v * c
    return out


def lowrank_features(Xn: np.ndarray, P: np.ndarray, pos: np.ndarray, pairs) -> np.ndarray:
    """x~_i = R_r(p_i) phi(P x_i) for one head: Xn [L, d], P [r, d] -> [L, r].

    Section 2.1: the normalised q/k are projected to rank r, passed through
    the pointwise map phi, and only then rotated (RoPE outside phi).
    Reading: one projection per layer shared by all heads, no bias.
    """
    return rope_rotate(phi_elu1(Xn @ P.T), pos, pairs)


def lowrank_state(kt: np.ndarray, V: np.ndarray) -> np.ndarray:
    """C = sum_j k~_j v_j^T over all tokens of one head: [r, d]."""
    return kt.T @ V


def lowrank_output(qt: np.ndarray, C: np.ndarray, eps: float = 1e-6, gamma=None) -> np.ndarray:
    """O_lr,i = RMSNorm(q~_i^T C) = gamma * y / sqrt(mean(y^2) + eps).

    Reading: no softmax-style denominator; eps = 1e-6 and gamma = 1 unless
    a weight is given.
    """
    y = qt @ C
    out = y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)
    if gamma is not None:
        out = out * np.asarray(gamma, dtype=np.float64)[None, :]
    return out


def gate_fuse(Os: np.ndarray, r: np.ndarray, g: np.ndarray, Olr: np.ndarray) -> np.ndarray:
    """O_i = O_s,i + g_i r_i O_lr,i (section 2.1, the O_i equation)."""
    return Os + (g * r)[:, None] * Olr


# ---------------------------------------------------------------------------
# The whole layer.
# ---------------------------------------------------------------------------

def rola_attention_head(Q, K, V, Qn, Kn, Pq, Pk, g, *, T, Hg, Wg, bq, bk, k_keep,
                        sm_scale, eps=1e-6, gamma=None, pairs=None):
    """RoLA attention for one (batch, head): every array float64, [L, ...].

    Returns a dict with the block map and every intermediate.
    """
    L, d = Q.shape
    rank = Pq.shape[0]
    if pairs is None:
        pairs = rope_pairs(rank)
    S = block_scores(Q, K, bq, bk)
    idx = topk_block_map(S, k_keep)
    Os, r = sparse_attention(Q, K, V, idx, bq, bk, sm_scale)
    pos = token_positions(T, Hg, Wg)
    qt = lowrank_features(Qn, Pq, pos, pairs)
    kt = lowrank_features(Kn, Pk, pos, pairs)
    C = lowrank_state(kt, V)
    Olr = lowrank_output(qt, C, eps, gamma)
    O = gate_fuse(Os, r, g, Olr)
    return dict(S=S, idx=idx, Os=Os, r=r, qt=qt, kt=kt, C=C, Olr=Olr, O=O)


def rola_attention(Qb, Kb, Vb, Pqb, Pkb, g, *, T, Hg, Wg, bq, bk, k_keep, sm_scale=None,
                   Qnb=None, Knb=None, eps=1e-6, heads=None):
    """Whole layer on bf16-bit inputs [B, L, H, d]; g float [B, L] (one gate
    per token, shared by the heads). Returns float64 arrays in [B, L, H, ...]
    layout for O, Os, Olr, r, and [B, H, ...] for idx and C.
    `heads` restricts the computation to a list of (b, h) pairs.
    """
    Bn, L, H, d = Qb.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    Pq = bf16_bits_to_f64(Pqb)
    Pk = bf16_bits_to_f64(Pkb)
    pairs = rope_pairs(Pq.shape[0])
    todo = heads if heads is not None else [(b, h) for b in range(Bn) for h in range(H)]
    res = {}
    for b, h in todo:
        Q = bf16_bits_to_f64(Qb[b, :, h])
        K = bf16_bits_to_f64(Kb[b, :, h])
        V = bf16_bits_to_f64(Vb[b, :, h])
        Qn = Q if Qnb is None else bf16_bits_to_f64(Qnb[b, :, h])
        Kn = K if Knb is None else bf16_bits_to_f64(Knb[b, :, h])
        res[(b, h)] = rola_attention_head(Q, K, V, Qn, Kn, Pq, Pk, np.asarray(g[b], dtype=np.float64),
                                          T=T, Hg=Hg, Wg=Wg, bq=bq, bk=bk, k_keep=k_keep,
                                          sm_scale=sm_scale, eps=eps, pairs=pairs)
    return res
