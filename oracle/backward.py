"""Backward of the RoLA attention layer (CPU oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

SparkDiffusion README_zh, distillation and operators sections: training the
sparse student needs a backward kernel for its sparse + low-rank attention
(the forward of the robotworld.top write-up, section 2.1). The pages
give no formulas for it; the backward is the exact derivative of the
forward as defined there, with the block map held fixed (top-k selection is
piecewise constant, so it passes no gradient).

Forward, one (batch, head), query i, key j (causal window optional):
  s_ij = scale q_i.k_j over the keys j of the kept blocks that i sees,
  p_ij = softmax_j(s_ij),  O_s,i = sum_j p_ij v_j,  r_i = RMS(O_s,i),
  a_i = P_q qn_i,  q~_i = R(p_i) phi(a_i),   b_j = P_k kn_j,  k~_j = R(p_j) phi(b_j),
  C_c = sum over the keys j chunk c sees of k~_j v_j^T,
  y_i = C_{c(i)}^T q~_i,  rho_i = sqrt(mean(y_i^2) + eps),  O_lr,i = w * y_i / rho_i,
  O_i = O_s,i + g_i r_i O_lr,i.

Backward, given dO (chain rule, step by step; every line is the derivative
of the forward line it names):
  dg_i = r_i (dO_i . O_lr,i)             dr_i = g_i (dO_i . O_lr,i)
  dO_lr,i = g_i r_i dO_i                 dO_s,i = dO_i + dr_i O_s,i / (d r_i)   (0 if r_i = 0)
  u_i = w * dO_lr,i,  dy_i = u_i / rho_i - y_i (u_i . y_i) / (d rho_i^3)
  dq~_i = C_{c(i)} dy_i,   dC_c = sum over queries i of chunk c of q~_i dy_i^T
  da_i = (R(p_i)^T dq~_i) * phi'(a_i),   dqn_i = P_q^T da_i,   dP_q = sum_i da_i qn_i^T
  dk~_j = (sum over chunks c that see j of dC_c) v_j,   dv_j += (same sum)^T k~_j
  db_j = (R(p_j)^T dk~_j) * phi'(b_j),   dkn_j = P_k^T db_j,   dP_k = sum_j db_j kn_j^T
  sparse branch: D_i = dO_s,i . O_s,i,  dp_ij = dO_s,i . v_j,  ds_ij = p_ij (dp_ij - D_i),
  dq_i = scale sum_j ds_ij k_j,  dk_j += scale sum_i ds_ij q_i,  dv_j += sum_i p_ij dO_s,i.
"""
from __future__ import annotations

import numpy as np

from .attention import block_ranges, phi_elu1, rope_pairs, rope_rotate, token_positions


def phi_elu1_grad(x: np.ndarray) -> np.ndarray:
    """phi'(x) for phi = ELU + 1: 1 for x > 0, exp(x) otherwise."""
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def rope_rotate_back(a: np.ndarray, pos: np.ndarray, pairs) -> np.ndarray:
    """R(p_i)^T applied to each row: the pair rotation by the negative angle."""
    out = a.copy()
    for dim, axis, theta in pairs:
        ang = pos[:, axis] * theta
        c, s = np.cos(ang), np.sin(ang)
        u, v = a[:, dim], a[:, dim + 1]
        out[:, dim] = u * c + v * s
        out[:, dim + 1] = -u * s + v * c
    return out


def sparse_attention_backward(Q, K, V, idx, bq, bk, sm_scale, dOs, M=None):
    """Gradients (dQ, dK, dV) of the block-sparse softmax branch for one head,
    and its output O_s, given dO_s. Same key sets as the forward
    (kept blocks, entries outside [0, Nk) keep nothing, M masks tokens)."""
    L, d = Q.shape
    kr = block_ranges(K.shape[0], bk)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    Os = np.zeros((L, d))
    for b, (s, e) in enumerate(block_ranges(L, bq)):
        blocks = [int(c) for c in idx[b] if 0 <= c < len(kr)]
        keys = np.concatenate([np.arange(*kr[c]) for c in blocks]) if blocks else np.zeros(0, dtype=np.int64)
        for i in range(s, e):
            ks = keys if M is None else keys[M[i, keys]]
            if ks.size == 0:
                continue
            sc = sm_scale * (K[ks] @ Q[i])
            p = np.exp(sc - sc.max())
            p /= p.sum()
            Os[i] = p @ V[ks]
            Di = dOs[i] @ Os[i]
            dp = V[ks] @ dOs[i]
            ds = p * (dp - Di)
            dQ[i] = sm_scale * (ds @ K[ks])
            np.add.at(dK, ks, sm_scale * ds[:, None] * Q[i][None, :])
            np.add.at(dV, ks, p[:, None] * dOs[i][None, :])
    return dQ, dK, dV, Os


def output_backward(dO, Os, r, Olr, g):
    """The fusion O = O_s + g r O_lr and r = RMS(O_s) backwards, per token:
    returns (dOs, dOlr, dg) for one head ([L, d], [L, d], [L])."""
    d = Os.shape[1]
    t = np.sum(dO * Olr, axis=1)
    dg = r * t
    dr = g * t
    dOlr = (g * r)[:, None] * dO
    safe_r = np.where(r > 0, r, 1.0)
    dOs = dO + np.where(r > 0, dr / (d * safe_r), 0.0)[:, None] * Os
    return dOs, dOlr, dg


def lowrank_query_backward(Qn, Pq, pos, pairs, C_tok, dOlr, eps=1e-6, gamma=None):
    """O_lr,i = w * y_i / rho_i, y_i = C_i^T q~_i, q~_i = R phi(P_q qn_i) backwards.

    C_tok: [L, r, d], the state each query uses. Returns (q~, dy, dq~, da,
    dqn): everything the state and projection gradients are built from.
    """
    d = Qn.shape[1]
    w = np.ones(d) if gamma is None else np.asarray(gamma, dtype=np.float64)
    a = Qn @ Pq.T
    qt = rope_rotate(phi_elu1(a), pos, pairs)
    y = np.einsum("ir,ird->id", qt, C_tok)
    rho = np.sqrt(np.mean(y * y, axis=1) + eps)
    u = w[None, :] * dOlr
    dy = u / rho[:, None] - y * (np.sum(u * y, axis=1) / (d * rho ** 3))[:, None]
    dqt = np.einsum("ird,id->ir", C_tok, dy)
    da = rope_rotate_back(dqt, pos, pairs) * phi_elu1_grad(a)
    return qt, dy, dqt, da, da @ Pq


def lowrank_key_backward(Kn, V, Pk, pos, pairs, dC_tok):
    """C = sum_j k~_j v_j^T, k~_j = R phi(P_k kn_j) backwards, given for each
    key the sum dC_tok [L, r, d] of the state gradients of the chunks that
    see it. Returns (dkn, dv, db) with dv the low-rank share of dV."""
    bpre = Kn @ Pk.T
    kt = rope_rotate(phi_elu1(bpre), pos, pairs)
    dkt = np.einsum("jrd,jd->jr", dC_tok, V)
    dv = np.einsum("jrd,jr->jd", dC_tok, kt)
    db = rope_rotate_back(dkt, pos, pairs) * phi_elu1_grad(bpre)
    return db @ Pk, dv, db


def rola_backward_head(Q, K, V, Qn, Kn, Pq, Pk, g, idx, dO, *, T, Hg, Wg, bq, bk, sm_scale,
                       chunk_tokens=0, window=0, eps=1e-6, gamma=None, pairs=None):
    """Forward intermediates and all gradients of one (batch, head).

    Q, K, V, Qn, Kn, dO: float64 [L, d]; Pq, Pk: [r, d]; g: [L]; idx: the
    fixed block map [Nq, k]. Returns a dict with O and dQ, dK, dV, dQn, dKn
    (the gradient reaching the low-rank inputs; add it to dQ / dK when the
    branch reads Q / K), dPq, dPk, dg ([L], this head's share of the gate
    gradient).
    """
    L, d = Q.shape
    if pairs is None:
        pairs = rope_pairs(Pq.shape[0])
    w = np.ones(d) if gamma is None else np.asarray(gamma, dtype=np.float64)
    ct = chunk_tokens if chunk_tokens > 0 else L
    c = np.arange(L) // ct
    M = None
    if chunk_tokens > 0:
        M = c[None, :] <= c[:, None]
        if window > 0:
            M &= c[None, :] > c[:, None] - window
    pos = token_positions(T, Hg, Wg)

    # forward (the sparse output comes with the backward below)
    a = Qn @ Pq.T
    qt = rope_rotate(phi_elu1(a), pos, pairs)
    bpre = Kn @ Pk.T
    kt = rope_rotate(phi_elu1(bpre), pos, pairs)
    n_ch = -(-L // ct)
    Mrow = (lambda s: np.ones(L, dtype=bool)) if M is None else (lambda s: M[s])
    C = np.stack([kt[Mrow(ch * ct)].T @ V[Mrow(ch * ct)] for ch in range(n_ch)])  # [n_ch, r, d]
    y = np.einsum("ir,ird->id", qt, C[c])
    rho = np.sqrt(np.mean(y * y, axis=1) + eps)
    Olr = w[None, :] * y / rho[:, None]

    # gate and RMS of the sparse output need O_s first: forward of the sparse
    # branch from the same routine (dO_s unknown yet, so a zero dO_s pass)
    _, _, _, Os = sparse_attention_backward(Q, K, V, idx, bq, bk, sm_scale, np.zeros((L, d)), M)
    r = np.sqrt(np.mean(Os * Os, axis=1))
    O = Os + (g * r)[:, None] * Olr

    # backward
    dOs, dOlr, dg = output_backward(dO, Os, r, Olr, g)
    _, dy, _, da, dQn = lowrank_query_backward(Qn, Pq, pos, pairs, C[c], dOlr, eps, gamma)
    dC = np.stack([qt[c == ch].T @ dy[c == ch] for ch in range(n_ch)])
    dPq = da.T @ Qn
    # key side: key j of chunk c' is seen by the queries of chunks c' .. c'+W-1
    # (every later chunk without a window)
    dC_seen = np.empty_like(dC)
    for ch in range(n_ch):
        last = n_ch - 1 if (chunk_tokens == 0 or window == 0) else min(n_ch - 1, ch + window - 1)
        dC_seen[ch] = dC[ch:last + 1].sum(axis=0)
    dKn, dV_lr, db = lowrank_key_backward(Kn, V, Pk, pos, pairs, dC_seen[c])
    dPk = db.T @ Kn
    dQ, dK, dV_s, _ = sparse_attention_backward(Q, K, V, idx, bq, bk, sm_scale, dOs, M)
    return dict(O=O, Os=Os, r=r, Olr=Olr, C=C, dC=dC, dOs=dOs, dQ=dQ, dK=dK, dV=dV_s + dV_lr, dQn=dQn, dKn=dKn,
                dPq=dPq, dPk=dPk, dg=dg)
