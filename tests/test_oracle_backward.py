"""Pins of the backward oracle (oracle/backward.py).

The backward is the derivative of the forward of the robotworld.top
write-up, section 2.1 (block map held fixed). It is tied to: central finite
differences of the FORWARD oracle (attention.py / variants.py, a separate
code path) on every input; PyTorch autograd through a float64 torch
restatement of the forward; and PyTorch's own attention backward
(scaled_dot_product_attention) for the sparse branch with all blocks kept.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import backward as ob

T_, HG, WG = 2, 4, 9  # 72 tokens: partial tail blocks at bq = 16, bk = 8
L = T_ * HG * WG
D, R = 8, 6  # rank 6: one RoPE pair on each axis
BQ, BK = 16, 8


def _case(seed, k=4):
    rng = np.random.default_rng(seed)
    X = {n: rng.standard_normal((L, D)) for n in ("Q", "K", "V", "Qn", "Kn", "dO")}
    X["Pq"] = rng.standard_normal((R, D)) / math.sqrt(D)
    X["Pk"] = rng.standard_normal((R, D)) / math.sqrt(D)
    X["g"] = 1.0 + rng.standard_normal(L)
    X["gamma"] = 1.0 + 0.2 * rng.standard_normal(D)
    nq, nk = -(-L // BQ), -(-L // BK)
    idx = np.stack([np.sort(rng.choice(nk, k, replace=False)) for _ in range(nq)]).astype(np.int32)
    return X, idx


def _forward(X, idx, chunk_tokens, window):
    """The forward oracle composed step by step with a fixed block map."""
    ct = chunk_tokens if chunk_tokens > 0 else L
    M = oracle.causal_window_mask(L, ct, window if chunk_tokens > 0 else 0)
    Os, r = oracle.sparse_attention_masked(X["Q"], X["K"], X["V"], idx, BQ, BK, 1 / math.sqrt(D), M)
    pos = oracle.token_positions(T_, HG, WG)
    pairs = oracle.rope_pairs(R)
    qt = oracle.lowrank_features(X["Qn"], X["Pq"], pos, pairs)
    kt = oracle.lowrank_features(X["Kn"], X["Pk"], pos, pairs)
    C = oracle.lowrank_states_masked(kt, X["V"], M, ct)
    Olr = np.empty((L, D))
    for c in range(C.shape[0]):
        s, e = c * ct, min(L, (c + 1) * ct)
        Olr[s:e] = oracle.lowrank_output(qt[s:e], C[c], 1e-6, X["gamma"])
    return oracle.gate_fuse(Os, r, X["g"], Olr)


def _backward(X, idx, chunk_tokens, window):
    return ob.rola_backward_head(X["Q"], X["K"], X["V"], X["Qn"], X["Kn"], X["Pq"], X["Pk"], X["g"], idx, X["dO"],
                                 T=T_, Hg=HG, Wg=WG, bq=BQ, bk=BK, sm_scale=1 / math.sqrt(D),
                                 chunk_tokens=chunk_tokens, window=window, gamma=X["gamma"])


GRADS = {"Q": "dQ", "K": "dK", "V": "dV", "Qn": "dQn", "Kn": "dKn", "Pq": "dPq", "Pk": "dPk", "g": "dg"}


@pytest.mark.parametrize("chunk,window", [(0, 0), (24, 0), (24, 2), (36, 1)])
def test_backward_equals_finite_differences_of_the_forward(chunk, window):
    X, idx = _case(1)
    res = _backward(X, idx, chunk, window)
    assert np.allclose(res["O"], _forward(X, idx, chunk, window), rtol=1e-12, atol=1e-12)
    loss = lambda Y: float(np.sum(X["dO"] * _forward(Y, idx, chunk, window)))
    rng = np.random.default_rng(2)
    h = 1e-6
    for name, gname in GRADS.items():
        flat = X[name].reshape(-1)
        for e in rng.choice(flat.size, 6, replace=False):
            Y = {k: v.copy() for k, v in X.items()}
            Y[name].reshape(-1)[e] += h
            up = loss(Y)
            Y[name].reshape(-1)[e] -= 2 * h
            dn = loss(Y)
            fd = (up - dn) / (2 * h)
            got = res[gname].reshape(-1)[e]
            assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd)), (name, e, got, fd)


def _torch_forward(T, idx, chunk_tokens, window):
    """The forward restated with float64 torch ops (dense masks), for autograd."""
    ct = chunk_tokens if chunk_tokens > 0 else L
    c = torch.arange(L) // ct
    M = c[None, :] <= c[:, None]
    if chunk_tokens > 0 and window > 0:
        M &= c[None, :] > c[:, None] - window
    keep = torch.zeros(L, L, dtype=torch.bool)
    for b in range(idx.shape[0]):
        for cc in idx[b]:
            if cc >= 0:
                keep[b * BQ:(b + 1) * BQ, cc * BK:(cc + 1) * BK] = True
    mask = M & keep
    s = (T["Q"] @ T["K"].T) / math.sqrt(D)
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=1).nan_to_num(0.0)
    Os = p @ T["V"]
    r = torch.sqrt((Os * Os).mean(dim=1))
    pos = torch.tensor(oracle.token_positions(T_, HG, WG), dtype=torch.float64)

    def feat(X, P):
        a = F.elu(X @ P.T) + 1.0
        cols = [a[:, i] for i in range(R)]
        for dim, axis, theta in oracle.rope_pairs(R):
            ang = pos[:, axis] * theta
            u, v = a[:, dim], a[:, dim + 1]
            cols[dim], cols[dim + 1] = u * torch.cos(ang) - v * torch.sin(ang), u * torch.sin(ang) + v * torch.cos(ang)
        return torch.stack(cols, dim=1)

    qt, kt = feat(T["Qn"], T["Pq"]), feat(T["Kn"], T["Pk"])
    y = ((qt @ kt.T) * M) @ T["V"]  # = q~_i^T C_{c(i)}, C over the keys i sees
    Olr = T["gamma"] * y / torch.sqrt((y * y).mean(dim=1, keepdim=True) + 1e-6)
    return Os + (T["g"] * r)[:, None] * Olr


@pytest.mark.parametrize("chunk,window", [(0, 0), (24, 2)])
def test_backward_equals_autograd(chunk, window):
    X, idx = _case(3, k=3)
    res = _backward(X, idx, chunk, window)
    T = {k: torch.tensor(v, requires_grad=(k in GRADS)) for k, v in X.items()}
    O = _torch_forward(T, idx, chunk, window)
    assert np.allclose(O.detach().numpy(), res["O"], rtol=1e-12, atol=1e-12)
    grads = torch.autograd.grad(O, [T[n] for n in GRADS], grad_outputs=T["dO"])
    for (name, gname), gt in zip(GRADS.items(), grads):
        assert np.allclose(res[gname], gt.numpy(), rtol=1e-10, atol=1e-11), name


def test_sparse_backward_all_blocks_is_library_attention_backward():
    rng = np.random.default_rng(4)
    Lq, d = 100, 16
    Q, K, V, dO = (rng.standard_normal((Lq, d)) for _ in range(4))
    idx = np.tile(np.arange(-(-Lq // 8)), (-(-Lq // 16), 1))
    dQ, dK, dV, Os = ob.sparse_attention_backward(Q, K, V, idx, 16, 8, 0.25, dO)
    Tq, Tk, Tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    out = F.scaled_dot_product_attention(Tq[None], Tk[None], Tv[None], scale=0.25)[0]
    gq, gk, gv = torch.autograd.grad(out, [Tq, Tk, Tv], grad_outputs=torch.tensor(dO))
    assert np.allclose(Os, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    for a, b in ((dQ, gq), (dK, gk), (dV, gv)):
        assert np.allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


def test_rotate_back_is_the_inverse_rotation():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((L, R))
    pos = oracle.token_positions(T_, HG, WG)
    pairs = oracle.rope_pairs(R)
    assert np.allclose(ob.rope_rotate_back(oracle.rope_rotate(a, pos, pairs), pos, pairs), a, atol=1e-13)


def test_phi_grad_closed_form():
    x = np.array([-3.0, -0.5, 0.0, 1e-9, 2.0])
    assert np.allclose(ob.phi_elu1_grad(x), [math.exp(-3.0), math.exp(-0.5), 1.0, 1.0, 1.0])
