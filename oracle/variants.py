"""Selector and autoregressive variants of RoLA attention (CPU oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

robotworld.top SparkDiffusion write-up, section 2.1: besides top-k over
block-level scores, the sparse branch A_M may keep its 1-s fraction of the
blocks by a fixed spatio-temporal pattern. Section 4 (ablations), on the
autoregressive extension: compensated sparse attention can be restricted to
a causal window, so that it serves chunk-by-chunk autoregressive video
diffusion.

Readings taken here (the pages give neither variant in more detail):
  * Fixed pattern: a query block keeps the k key blocks whose centroids in
    latent (t, h, w) coordinates lie nearest to its own centroid (squared
    Euclidean distance, unit grid spacing on every axis, no data involved);
    ties go to the lower block index, as for the scored top-k.
  * Causal window: tokens form autoregressive chunks of `chunk_tokens`
    consecutive raster tokens (a chunk of latent frames is
    frames * Hg * Wg tokens). A query in chunk c sees every key of chunks
    c - window + 1 .. c (window 0: every chunk up to c), and nothing later.
    Inside a chunk attention stays bidirectional.
  * Both branches are restricted: the sparse branch keeps only key blocks
    that hold at least one key some query of the block may see, and masks
    the rest token by token; the low-rank state of a query sums k~ v^T over
    exactly the keys it sees. A query that sees no key of its kept blocks
    gets a zero sparse output (and r = 0).
  * When fewer than k key blocks are allowed for a query block, all allowed
    blocks are kept and the row is padded with -1 (no block).
"""
from __future__ import annotations

import numpy as np

from .attention import (
    block_ranges,
    dense_attention,
    block_scores,
    lowrank_features,
    lowrank_output,
    gate_fuse,
    rope_pairs,
    token_positions,
)


# ---------------------------------------------------------------------------
# Fixed spatio-temporal selector.
# ---------------------------------------------------------------------------

def block_centroids(L: int, bs: int, T: int, Hg: int, Wg: int) -> np.ndarray:
    """Mean latent position (t, h, w) of the valid tokens of each block: [n, 3].

    The integer coordinate sums are exact; each mean is one float64 division.
    """
    pos = token_positions(T, Hg, Wg)
    assert pos.shape[0] == L
    out = []
    for s, e in block_ranges(L, bs):
        sums = pos[s:e].sum(axis=0)  # int64, exact
        out.append([float(sums[a]) / float(e - s) for a in range(3)])
    return np.array(out, dtype=np.float64)


def fixed_block_scores(L: int, bq: int, bk: int, T: int, Hg: int, Wg: int) -> np.ndarray:
    """S[b, c] = -|centroid(query block b) - centroid(key block c)|^2.

    Evaluated as -((dt*dt + dh*dh) + dw*dw) in float64 without fused
    multiply-adds, so that the order of the sums is fixed.
    """
    cq = block_centroids(L, bq, T, Hg, Wg)
    ck = block_centroids(L, bk, T, Hg, Wg)
    d = cq[:, None, :] - ck[None, :, :]
    sq = d * d
    return -((sq[..., 0] + sq[..., 1]) + sq[..., 2])


# ---------------------------------------------------------------------------
# Causal window.
# ---------------------------------------------------------------------------

def causal_window_mask(L: int, chunk_tokens: int, window: int) -> np.ndarray:
    """M[i, j] = query i may see key j (bool [L, L])."""
    c = np.arange(L) // chunk_tokens
    M = c[None, :] <= c[:, None]
    if window > 0:
        M &= c[None, :] > c[:, None] - window
    return M


def block_allowed(M: np.ndarray, bq: int, bk: int) -> np.ndarray:
    """A[b, c] = some query of block b may see some key of block c."""
    L = M.shape[0]
    qr, kr = block_ranges(L, bq), block_ranges(M.shape[1], bk)
    A = np.zeros((len(qr), len(kr)), dtype=bool)
    for b, (qs, qe) in enumerate(qr):
        for c, (ks, ke) in enumerate(kr):
            A[b, c] = M[qs:qe, ks:ke].any()
    return A


def topk_block_map_allowed(S: np.ndarray, k: int, allowed: np.ndarray) -> np.ndarray:
    """Top-k of each row of S among its allowed columns, ascending, -1 padded.

    Order by score (descending), then by block index; the first min(k, n)
    allowed columns are kept.
    """
    n_rows, n_cols = S.shape
    out = np.full((n_rows, k), -1, dtype=np.int32)
    for b in range(n_rows):
        cols = np.nonzero(allowed[b])[0]
        order = cols[np.lexsort((cols, -S[b, cols]))]
        kept = np.sort(order[:k])
        out[b, : len(kept)] = kept
    return out


def sparse_attention_masked(Q, K, V, idx, bq: int, bk: int, sm_scale: float, M=None):
    """Block-sparse softmax attention for one head under a token mask.

    Query i of block b attends to the keys of the kept blocks idx[b] (entries
    outside [0, Nk) keep nothing) that M[i] allows (M None: all). A query
    with no such key gets a zero row. Returns (O_s, r) as sparse_attention.
    """
    L, d = Q.shape
    kr = block_ranges(K.shape[0], bk)
    Os = np.zeros((L, d))
    for b, (s, e) in enumerate(block_ranges(L, bq)):
        blocks = [int(c) for c in idx[b] if 0 <= c < len(kr)]
        keys = np.concatenate([np.arange(*kr[c]) for c in blocks]) if blocks else np.zeros(0, dtype=np.int64)
        for i in range(s, e):
            ks = keys if M is None else keys[M[i, keys]]
            if ks.size:
                Os[i] = dense_attention(Q[i : i + 1], K[ks], V[ks], sm_scale)[0]
    r = np.sqrt(np.mean(Os * Os, axis=1))
    return Os, r


def lowrank_states_masked(kt: np.ndarray, V: np.ndarray, M: np.ndarray, chunk_tokens: int) -> np.ndarray:
    """State of every autoregressive chunk: C_c = sum over the keys j that the
    queries of chunk c see of k~_j v_j^T; [n_chunks, r, d]. All queries of a
    chunk see the same keys, so the first query's row of M stands for it.
    """
    L = M.shape[0]
    out = []
    for s in range(0, L, chunk_tokens):
        sel = M[s]
        out.append(kt[sel].T @ V[sel])
    return np.stack(out)


def rola_attention_head_variant(Q, K, V, Qn, Kn, Pq, Pk, g, *, T, Hg, Wg, bq, bk, k_keep, sm_scale,
                                select="topk", chunk_tokens=0, window=0, eps=1e-6, gamma=None, pairs=None):
    """RoLA attention for one (batch, head) with a selector and an optional
    causal window (chunk_tokens 0: bidirectional). Same returns as
    rola_attention_head, with C per autoregressive chunk [n_chunks, r, d].
    """
    L, d = Q.shape
    if pairs is None:
        pairs = rope_pairs(Pq.shape[0])
    ct = chunk_tokens if chunk_tokens > 0 else L
    M = causal_window_mask(L, ct, window if chunk_tokens > 0 else 0)
    if select == "topk":
        S = block_scores(Q, K, bq, bk)
    elif select == "fixed":
        S = fixed_block_scores(L, bq, bk, T, Hg, Wg)
    else:
        raise ValueError(select)
    idx = topk_block_map_allowed(S, k_keep, block_allowed(M, bq, bk))
    Os, r = sparse_attention_masked(Q, K, V, idx, bq, bk, sm_scale, M)
    pos = token_positions(T, Hg, Wg)
    qt = lowrank_features(Qn, Pq, pos, pairs)
    kt = lowrank_features(Kn, Pk, pos, pairs)
    C = lowrank_states_masked(kt, V, M, ct)
    Olr = np.empty((L, d))
    for c in range(C.shape[0]):
        s, e = c * ct, min(L, (c + 1) * ct)
        Olr[s:e] = lowrank_output(qt[s:e], C[c], eps, gamma)
    O = gate_fuse(Os, r, g, Olr)
    return dict(S=S, idx=idx, Os=Os, r=r, qt=qt, kt=kt, C=C, Olr=Olr, O=O, M=M)
