"""GPU parity of the backward of the fused layer against the oracle.

The HIP backward (sd_rola_backward, through the C ABI) and the oracle's
chain-rule backward (oracle/backward.py, pinned by finite differences of
the forward oracle) run on the same seeded inputs and the same block map
(the one the GPU forward chose).

Tolerance, from the arithmetic: the softmax branch feeds P, dS and dO_s to
the matrix cores as bf16 (as attention backward kernels do), each rounded to
nearest with a relative error of at most 2^-9; every gradient element is a
sum of products that carry one or two such roundings, so its relative L2
error is of order 2^-9. The low-rank products use hi/lo bf16 splits (about
16 bits) and f32 sums. Each of dQ, dK, dV, dQn, dKn is held to a relative
L2 error of 2^-7 (4 x 2^-9) and a worst element of 2^-6 of its largest
magnitude; dPq, dPk and dg, whose errors come from the same roundings
averaged over every token, to a relative L2 error of 2^-9. Measured worst:
2.5e-3, 3.7e-3 and 4.0e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from workloads import synthetic
from gpu_util import dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu

RAGGED = synthetic.AttnConfig("ragged-330", 1, 3, 128, 3, 10, 11, 128, 64, 0.70, 32)
RAGGED64 = synthetic.AttnConfig("ragged-d64", 2, 2, 64, 5, 7, 13, 64, 64, 0.60, 16)
FRAMES = synthetic.AttnConfig("frames-780", 1, 2, 128, 6, 10, 13, 128, 64, 0.70, 32)
MID = synthetic.AttnConfig("mid-2176", 1, 2, 128, 2, 32, 34, 128, 64, 0.90, 32)


def _rel(got, ref, name, rel_l2=2.0 ** -7, max_frac=2.0 ** -6):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), name
    scale = max(np.abs(ref).max(), 1e-30)
    ma = np.abs(got - ref).max() / scale
    rl = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"  {name}: rel_l2={rl:.2e} max_abs/max|ref|={ma:.2e}")
    assert rl <= rel_l2 and ma <= max_frac, f"{name}: rel_l2 {rl:.3e}, max {ma:.3e}"


def _run(cfg, seed=0, chunk_frames=0, window=0, separate_qk=False, per_head_gate=False, batch_shared_gate=False,
         rms_weight=False, per_head_proj=False):
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, seed)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    if per_head_proj:  # one P_q, P_k per head: [H, rank, d]
        pp = [synthetic.gen_lowrank_params(cfg, seed=11 + hh) for hh in range(cfg.H)]
        Pqb, Pkb = np.stack([x[0] for x in pp]), np.stack([x[1] for x in pp])
    rng = np.random.default_rng(seed + 100)
    if per_head_gate:
        g = (1.0 + rng.standard_normal((cfg.B, cfg.L, cfg.H))).astype(np.float32)
    else:
        g = synthetic.gen_gate(cfg, amplified=True)
    if batch_shared_gate:  # one gate row read by every batch element
        g = np.broadcast_to(g[:1], g.shape).copy()
    dOb = synthetic.f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.L, cfg.H, cfg.d)).astype(np.float32))
    Qnb = Knb = None
    if separate_qk:
        Qnb, Knb, _ = synthetic.gen_qkv(cfg, seed + 7)
    ct = chunk_frames * cfg.Hg * cfg.Wg
    var = dict(chunk_tokens=ct, window=window)
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    Q, K, V, dO = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_bf16(dOb)
    Qn = dev_bf16(Qnb) if separate_qk else None
    Kn = dev_bf16(Knb) if separate_qk else None
    wb = synthetic.gen_norm_weight(cfg.d, seed) if rms_weight else None
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb), rms_weight=dev_bf16(wb) if rms_weight else None,
                          head_stride=cfg.rank * cfg.d if per_head_proj else 0)
    k = oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))
    nq = -(-cfg.L // cfg.block_q)
    idx = torch.empty((cfg.B, cfg.H, nq, k), dtype=torch.int32, device="cuda")
    gd = dev_f32(g[:1]).expand(g.shape) if batch_shared_gate else dev_f32(g)
    ws = sd.rola_workspace(Q, lr, k, grid=grid, block_q=cfg.block_q, **var)
    sd.sd_rola_prepare(Q, K, V, lr, k, ws, grid=grid, block_q=cfg.block_q, Qn=Qn, Kn=Kn, idx_out=idx, **var)
    grads = sd.sd_rola_backward(Q, K, V, gd, lr, k, idx, dO, grid=grid, block_q=cfg.block_q, Qn=Qn, Kn=Kn, **var)
    torch.cuda.synchronize()
    got = {n: (host(t) if t is not None else None) for n, t in grads.items()}
    idx = idx.cpu().numpy()
    f = oracle.bf16_bits_to_f64
    Pq_all, Pk_all = f(Pqb), f(Pkb)
    ref = {"dPq": 0.0, "dPk": 0.0, "dg": np.zeros(g.shape)}
    if per_head_proj:
        ref["dPq"] = np.zeros((cfg.H, cfg.rank, cfg.d))
        ref["dPk"] = np.zeros((cfg.H, cfg.rank, cfg.d))
    for b in range(cfg.B):
        for h in range(cfg.H):
            Pq, Pk = (Pq_all[h], Pk_all[h]) if per_head_proj else (Pq_all, Pk_all)
            X = [f(x[b, :, h]) for x in (Qb, Kb, Vb)]
            Xn = [f(Qnb[b, :, h]), f(Knb[b, :, h])] if separate_qk else X[:2]
            gh = (g[b, :, h] if per_head_gate else g[b]).astype(np.float64)
            res = oracle.rola_backward_head(*X, *Xn, Pq, Pk, gh, idx[b, h], f(dOb[b, :, h]), T=cfg.T, Hg=cfg.Hg,
                                            Wg=cfg.Wg, bq=cfg.block_q, bk=cfg.block_k,
                                            sm_scale=1.0 / math.sqrt(cfg.d), chunk_tokens=ct, window=window,
                                            gamma=f(wb) if rms_weight else None)
            dQ, dK = res["dQ"], res["dK"]
            if separate_qk:
                _rel(got["dQn"][b, :, h], res["dQn"], f"dQn b{b} h{h}")
                _rel(got["dKn"][b, :, h], res["dKn"], f"dKn b{b} h{h}")
            else:
                dQ, dK = dQ + res["dQn"], dK + res["dKn"]
            _rel(got["dQ"][b, :, h], dQ, f"dQ b{b} h{h}")
            _rel(got["dK"][b, :, h], dK, f"dK b{b} h{h}")
            _rel(got["dV"][b, :, h], res["dV"], f"dV b{b} h{h}")
            if per_head_proj:
                ref["dPq"][h] += res["dPq"][: cfg.rank]
                ref["dPk"][h] += res["dPk"][: cfg.rank]
            else:
                ref["dPq"] = ref["dPq"] + res["dPq"]
                ref["dPk"] = ref["dPk"] + res["dPk"]
            if per_head_gate:
                ref["dg"][b, :, h] = res["dg"]
            else:
                ref["dg"][b] += res["dg"]
    if per_head_proj:
        for h in range(cfg.H):
            _rel(got["dPq"][h], ref["dPq"][h], f"dPq h{h}", rel_l2=2.0 ** -9)
            _rel(got["dPk"][h], ref["dPk"][h], f"dPk h{h}", rel_l2=2.0 ** -9)
    else:
        _rel(got["dPq"], ref["dPq"][: cfg.rank], "dPq", rel_l2=2.0 ** -9)
        _rel(got["dPk"], ref["dPk"][: cfg.rank], "dPk", rel_l2=2.0 ** -9)
    if batch_shared_gate:  # the gradient of the shared row sums over the batch
        assert grads["dg"].stride(0) == 0
        ref["dg"] = ref["dg"].sum(axis=0, keepdims=True)
        got["dg"] = got["dg"][:1]
    _rel(got["dg"], ref["dg"], "dg", rel_l2=2.0 ** -9)
    return grads


@pytest.mark.parametrize("cfg", [RAGGED, RAGGED64, MID], ids=lambda c: c.name)
def test_backward_bidirectional(cfg):
    say(f"backward {cfg.name}")
    _run(cfg)


def test_backward_gate_shared_by_the_batch():
    # B = 2 with one gate row broadcast over the batch (stride 0): dg sums the
    # two batch elements' gradients instead of keeping one of them
    say("backward ragged-d64, gate broadcast over the batch")
    _run(RAGGED64, seed=4, batch_shared_gate=True)


@pytest.mark.parametrize("cfg", [RAGGED, RAGGED64], ids=lambda c: c.name)
def test_backward_rms_weight(cfg):
    # a non-trivial RMSNorm weight on the low-rank output: it enters dg, dy
    # and the RMS coupling term of dO_s
    say(f"backward {cfg.name} with an RMSNorm weight")
    _run(cfg, seed=6, rms_weight=True)


@pytest.mark.parametrize("cfg", [RAGGED, RAGGED64], ids=lambda c: c.name)
def test_backward_per_head_projections(cfg):
    # one P_q and P_k per head (P_head_stride = rank * d): dP_q, dP_k are
    # then per head, each summed over that head's tokens (and the batch)
    say(f"backward {cfg.name} with per-head projections")
    _run(cfg, seed=8, per_head_proj=True)


def test_backward_separate_qk_and_per_head_gate():
    say("backward ragged, separate Qn/Kn, per-head gate")
    _run(RAGGED, seed=3, separate_qk=True, per_head_gate=True)


@pytest.mark.parametrize("frames,window", [(1, 0), (1, 2), (2, 1)])
def test_backward_causal_window(frames, window):
    say(f"backward frames-780 causal f{frames} w{window}")
    _run(FRAMES, seed=1, chunk_frames=frames, window=window)


def test_backward_d64_causal():
    say("backward ragged-d64 causal f1 w2")
    _run(RAGGED64, seed=2, chunk_frames=1, window=2)


def test_backward_deterministic():
    a = _run(RAGGED, seed=5)
    b = _run(RAGGED, seed=5)
    for n in ("dQ", "dK", "dV", "dPq", "dPk", "dg"):
        assert torch.equal(a[n], b[n]), n


def test_backward_720p_sampled():
    # the 720P layer as the benchmark runs it; the oracle composes its
    # backward pieces for one head: every query's forward and low-rank
    # quantities (the state gradient sums over all of them), then the sparse
    # branch's dQ of sampled query blocks and dK / dV of sampled key blocks
    # from exactly the query blocks that keep them
    cfg = synthetic.WAN14B_720P
    say("backward 720p: generating inputs")
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 0)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    g = synthetic.gen_gate(cfg, amplified=True)
    dOb = synthetic.f32_to_bf16_bits(
        np.random.default_rng(9).standard_normal((cfg.B, cfg.L, cfg.H, cfg.d)).astype(np.float32))
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    Q, K, V, dO = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_bf16(dOb)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    k = oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))
    nq, nk = -(-cfg.L // cfg.block_q), -(-cfg.L // cfg.block_k)
    idx = torch.empty((1, cfg.H, nq, k), dtype=torch.int32, device="cuda")
    ws = sd.rola_workspace(Q, lr, k, grid=grid)
    sd.sd_rola_prepare(Q, K, V, lr, k, ws, grid=grid, idx_out=idx)
    say("  running sd_rola_backward")
    grads = sd.sd_rola_backward(Q, K, V, dev_f32(g), lr, k, idx, dO, grid=grid)
    torch.cuda.synchronize()
    heads = (23,)
    got = {n: grads[n][0, :, list(heads)].cpu().numpy().astype(np.float64) for n in ("dQ", "dK", "dV")}
    idx = idx.cpu().numpy()
    del grads, ws, Q, K, V, dO
    f = oracle.bf16_bits_to_f64
    Pq, Pk = f(Pqb), f(Pkb)
    pos = oracle.token_positions(cfg.T, cfg.Hg, cfg.Wg)
    pairs = oracle.rope_pairs(cfg.rank)
    scale = 1.0 / math.sqrt(cfg.d)
    rng = np.random.default_rng(2)
    for hi, h in enumerate(heads):
        Qh, Kh, Vh, dOh = (f(x[0, :, h]) for x in (Qb, Kb, Vb, dOb))
        mh = idx[0, h]
        Os, r = oracle.sparse_attention(Qh, Kh, Vh, mh, cfg.block_q, cfg.block_k, scale)
        qt = oracle.lowrank_features(Qh, Pq, pos, pairs)
        kt = oracle.lowrank_features(Kh, Pk, pos, pairs)
        C = oracle.lowrank_state(kt, Vh)
        Olr = oracle.lowrank_output(qt, C, 1e-6)
        dOs, dOlr, _ = oracle.output_backward(dOh, Os, r, Olr, g[0].astype(np.float64))
        Ct = np.broadcast_to(C, (cfg.L,) + C.shape)
        qt, dy, _, _, dQn = oracle.lowrank_query_backward(Qh, Pq, pos, pairs, Ct, dOlr)
        dC = qt.T @ dy
        dKn, dv_lr, _ = oracle.lowrank_key_backward(Kh, Vh, Pk, pos, pairs, np.broadcast_to(dC, (cfg.L,) + dC.shape))
        for qb in sorted(set(rng.choice(nq - 1, 4, replace=False).tolist()) | {nq - 1}):
            s0, e0 = qb * cfg.block_q, min(cfg.L, (qb + 1) * cfg.block_q)
            dQs, _, _, _ = oracle.sparse_attention_backward(Qh[s0:e0], Kh, Vh, mh[qb:qb + 1], cfg.block_q,
                                                            cfg.block_k, scale, dOs[s0:e0])
            _rel(got["dQ"][s0:e0, hi], dQs + dQn[s0:e0], f"dQ head {h} query block {qb}")
        # key blocks kept by at most 40 query blocks (the oracle walks every
        # query of every one of them; the partial tail block and the longest
        # lists are covered by the smaller cases)
        counts = np.bincount(mh.ravel(), minlength=nk)
        cands = np.nonzero((counts > 0) & (counts <= 40))[0]
        for c in sorted(set(rng.choice(cands, 3, replace=False).tolist()) | {int(cands[counts[cands].argmax()])}):
            keep = [qb for qb in range(nq) if c in mh[qb]]
            rows = np.concatenate([np.arange(qb * cfg.block_q, min(cfg.L, (qb + 1) * cfg.block_q)) for qb in keep])
            _, dKs, dVs, _ = oracle.sparse_attention_backward(Qh[rows], Kh, Vh, mh[keep], cfg.block_q, cfg.block_k,
                                                             scale, dOs[rows])
            s0, e0 = c * cfg.block_k, min(cfg.L, (c + 1) * cfg.block_k)
            _rel(got["dK"][s0:e0, hi], dKs[s0:e0] + dKn[s0:e0], f"dK head {h} key block {c} ({len(keep)} q-blocks)")
            _rel(got["dV"][s0:e0, hi], dVs[s0:e0] + dv_lr[s0:e0], f"dV head {h} key block {c}")


@pytest.mark.parametrize("frames,window", [(0, 0), (1, 2)])
def test_backward_with_saved_forward_is_identical(frames, window):
    # a training step keeps O_s, its RMS and the log-sum-exp in the forward;
    # the backward then skips the sparse recomputation and must give the same
    # bits, and the saving forward the same output
    cfg = FRAMES
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 4)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    g = synthetic.gen_gate(cfg, amplified=True)
    dOb = synthetic.f32_to_bf16_bits(
        np.random.default_rng(5).standard_normal((cfg.B, cfg.L, cfg.H, cfg.d)).astype(np.float32))
    var = dict(chunk_tokens=frames * cfg.Hg * cfg.Wg, window=window)
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    Q, K, V, dO, gd = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_bf16(dOb), dev_f32(g)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    k = oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))
    idx = torch.empty((1, cfg.H, -(-cfg.L // cfg.block_q), k), dtype=torch.int32, device="cuda")
    ws = sd.rola_workspace(Q, lr, k, grid=grid, **var)
    sd.sd_rola_prepare(Q, K, V, lr, k, ws, grid=grid, idx_out=idx, **var)
    save = sd.SavedForward(Q)
    O1 = sd.sd_rola_apply(Q, K, V, gd, lr, k, ws, grid=grid, idx=idx, save=save, **var)
    O2 = sd.sd_rola_apply(Q, K, V, gd, lr, k, ws, grid=grid, idx=idx, **var)
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    g1 = sd.sd_rola_backward(Q, K, V, gd, lr, k, idx, dO, grid=grid, saved=save, **var)
    g2 = sd.sd_rola_backward(Q, K, V, gd, lr, k, idx, dO, grid=grid, **var)
    torch.cuda.synchronize()
    for n in ("dQ", "dK", "dV", "dPq", "dPk", "dg"):
        assert torch.equal(g1[n], g2[n]), n
    # the kept O_s and RMS against the oracle's sparse branch
    idx_np = idx.cpu().numpy()
    ct = var["chunk_tokens"] or cfg.L
    M = oracle.causal_window_mask(cfg.L, ct, window)
    for h in range(cfg.H):
        f = oracle.bf16_bits_to_f64
        Os, r = oracle.sparse_attention_masked(f(Qb[0, :, h]), f(Kb[0, :, h]), f(Vb[0, :, h]), idx_np[0, h],
                                               cfg.block_q, cfg.block_k, 1.0 / math.sqrt(cfg.d), M)
        _rel(host(save.Os[0, :, h]), Os, f"saved O_s h{h}")
        _rel(host(save.rms[0, :, h]), r, f"saved rms h{h}")
        assert torch.isfinite(save.lse[0, h]).all()
