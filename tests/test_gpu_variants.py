"""GPU parity of the selector and causal-window variants against the oracle.

robotworld.top SparkDiffusion write-up, section 2.1 (the fixed
spatio-temporal pattern as selector) and section 4 (compensated sparse
attention restricted to a causal window). The HIP path runs through the C
ABI on seeded inputs. The fixed pattern's block map is computed from the
same float64 operations on both sides and must match bit for bit; the scored
map under a causal window must match outside the tie window, with identical
-1 padding; float outputs are held to the bounds of the bidirectional path
(max-abs 2e-2, relative L2 1e-2). Chunks are whole latent frames whose
token counts are not multiples of the 64-key or 128-query blocks, so blocks
and waves straddle chunk boundaries.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from workloads import synthetic
from gpu_util import TIE_REL, assert_close, dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu

FRAMES = synthetic.AttnConfig("frames-780", 1, 2, 128, 6, 10, 13, 128, 64, 0.70, 32)
FRAMES64 = synthetic.AttnConfig("frames-d64", 2, 2, 64, 5, 7, 13, 64, 64, 0.60, 16)
MID2 = synthetic.AttnConfig("mid-2176", 1, 4, 128, 2, 32, 34, 128, 64, 0.90, 32)

# (config, frames per chunk, window in chunks); frames 0 = bidirectional
CAUSAL = [(FRAMES, 1, 0), (FRAMES, 1, 2), (FRAMES, 2, 1), (FRAMES64, 1, 3), (FRAMES64, 2, 0), (MID2, 1, 0)]


def _id(case):
    cfg, fr, w = case
    return f"{cfg.name}-f{fr}-w{w}"


def _f(bits, b, h):
    return oracle.bf16_bits_to_f64(bits[b, :, h])


def _kkeep(cfg):
    return oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))


def _mask(cfg, frames, window):
    ct = frames * cfg.Hg * cfg.Wg if frames else cfg.L
    return ct, oracle.causal_window_mask(cfg.L, ct, window if frames else 0)


def _map_diff(idx, S, k, allowed):
    """Blocks in one map and not the other, outside the tie window at the
    k-th largest allowed score; the -1 padding must agree exactly."""
    ref = oracle.topk_block_map_allowed(S, k, allowed)
    mism = rows = 0
    for b in range(S.shape[0]):
        g = idx[b]
        n = int((ref[b] >= 0).sum())
        assert (g[n:] == -1).all() and (g[:n] >= 0).all(), f"row {b}: padding {g} vs {ref[b]}"
        assert (np.diff(g[:n]) > 0).all(), f"row {b} not ascending: {g}"
        assert allowed[b, g[:n]].all(), f"row {b} keeps a block outside the window"
        if np.array_equal(g, ref[b]):
            continue
        rows += 1
        sc = np.sort(S[b, allowed[b]])[::-1]
        tau = sc[k - 1] if sc.size >= k else -np.inf
        for c in set(g[:n].tolist()) ^ set(ref[b, :n].tolist()):
            if not abs(S[b, c] - tau) <= TIE_REL * max(1.0, abs(tau)):
                mism += 1
    return mism, rows


@pytest.mark.parametrize("cfg", [synthetic.TINY, FRAMES, FRAMES64, synthetic.WAN14B_720P], ids=lambda c: c.name)
def test_fixed_block_map_bit_exact(cfg):
    say(f"fixed block map {cfg.name}")
    k = _kkeep(cfg)
    Q = torch.zeros((cfg.B, cfg.L, cfg.H, cfg.d), dtype=torch.bfloat16, device="cuda")
    idx = sd.sd_block_select(Q, Q, k, block_q=cfg.block_q, block_k=cfg.block_k, grid=(cfg.T, cfg.Hg, cfg.Wg),
                             select="fixed").cpu().numpy()
    S = oracle.fixed_block_scores(cfg.L, cfg.block_q, cfg.block_k, cfg.T, cfg.Hg, cfg.Wg)
    ref = oracle.topk_block_map_allowed(S, k, np.ones_like(S, dtype=bool))
    assert (idx == ref[None, None]).all()


@pytest.mark.parametrize("case", CAUSAL, ids=_id)
@pytest.mark.parametrize("select", ["topk", "fixed"])
def test_causal_block_map(case, select):
    cfg, frames, window = case
    say(f"causal block map {_id(case)} {select}")
    Qb, Kb, _ = synthetic.gen_qkv(cfg, 0)
    k = _kkeep(cfg)
    ct, M = _mask(cfg, frames, window)
    allowed = oracle.block_allowed(M, cfg.block_q, cfg.block_k)
    idx = sd.sd_block_select(dev_bf16(Qb), dev_bf16(Kb), k, block_q=cfg.block_q, block_k=cfg.block_k,
                             grid=(cfg.T, cfg.Hg, cfg.Wg), select=select, chunk_tokens=ct,
                             window=window).cpu().numpy()
    for b in range(cfg.B):
        for h in range(cfg.H):
            if select == "fixed":
                S = oracle.fixed_block_scores(cfg.L, cfg.block_q, cfg.block_k, cfg.T, cfg.Hg, cfg.Wg)
                assert (idx[b, h] == oracle.topk_block_map_allowed(S, k, allowed)).all()
            else:
                S = oracle.block_scores(_f(Qb, b, h), _f(Kb, b, h), cfg.block_q, cfg.block_k)
                mism, _ = _map_diff(idx[b, h], S, k, allowed)
                assert mism == 0


def test_causal_block_map_short_rows_padded():
    # one-frame chunks without history and k above the allowed count: the
    # early query blocks keep every allowed block and end in -1
    cfg = FRAMES
    k = 6
    ct = cfg.Hg * cfg.Wg
    Q = torch.zeros((1, cfg.L, cfg.H, cfg.d), dtype=torch.bfloat16, device="cuda")
    idx = sd.sd_block_select(Q, Q, k, block_q=128, block_k=64, grid=(cfg.T, cfg.Hg, cfg.Wg), select="fixed",
                             chunk_tokens=ct, window=1).cpu().numpy()
    M = oracle.causal_window_mask(cfg.L, ct, 1)
    allowed = oracle.block_allowed(M, 128, 64)
    S = oracle.fixed_block_scores(cfg.L, 128, 64, cfg.T, cfg.Hg, cfg.Wg)
    ref = oracle.topk_block_map_allowed(S, k, allowed)
    assert (ref == -1).any()
    assert (idx == ref[None, None]).all()


def _oracle_maps(cfg, Qb, Kb, k, M, select="topk"):
    allowed = oracle.block_allowed(M, cfg.block_q, cfg.block_k)
    maps = np.zeros((cfg.B, cfg.H, -(-cfg.L // cfg.block_q), k), dtype=np.int32)
    for b in range(cfg.B):
        for h in range(cfg.H):
            S = (oracle.block_scores(_f(Qb, b, h), _f(Kb, b, h), cfg.block_q, cfg.block_k) if select == "topk" else
                 oracle.fixed_block_scores(cfg.L, cfg.block_q, cfg.block_k, cfg.T, cfg.Hg, cfg.Wg))
            maps[b, h] = oracle.topk_block_map_allowed(S, k, allowed)
    return maps


@pytest.mark.parametrize("case", CAUSAL, ids=_id)
def test_causal_sparse_attn(case):
    cfg, frames, window = case
    say(f"causal sparse attn {_id(case)}")
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 1)
    k = _kkeep(cfg)
    ct, M = _mask(cfg, frames, window)
    maps = _oracle_maps(cfg, Qb, Kb, k, M)
    Os, rms = sd.sd_sparse_attn(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), torch.from_numpy(maps).cuda(),
                                block_q=cfg.block_q, chunk_tokens=ct, window=window)
    Os, rms = host(Os), host(rms)
    scale = 1.0 / math.sqrt(cfg.d)
    for b in range(cfg.B):
        for h in range(cfg.H):
            ref, r = oracle.sparse_attention_masked(_f(Qb, b, h), _f(Kb, b, h), _f(Vb, b, h), maps[b, h],
                                                    cfg.block_q, cfg.block_k, scale, M)
            assert_close(Os[b, :, h], ref, f"O_s b{b} h{h}")
            assert_close(rms[b, :, h], r, f"rms b{b} h{h}")


def test_causal_sparse_rows_that_see_nothing_are_zero():
    # query block 1 holds tokens 128..255: 128, 129 end chunk 0 (130 tokens),
    # the rest are chunk 1; with window 1 and only key block 0 kept, the
    # queries of chunk 1 see no kept key
    cfg = FRAMES
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 2)
    ct = cfg.Hg * cfg.Wg
    nq = -(-cfg.L // cfg.block_q)
    maps = np.full((1, cfg.H, nq, 2), -1, dtype=np.int32)
    maps[..., 0] = 0
    Os, rms = sd.sd_sparse_attn(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), torch.from_numpy(maps).cuda(),
                                block_q=128, chunk_tokens=ct, window=1)
    Os, rms = host(Os), host(rms)
    M = oracle.causal_window_mask(cfg.L, ct, 1)
    for h in range(cfg.H):
        ref, r = oracle.sparse_attention_masked(_f(Qb, 0, h), _f(Kb, 0, h), _f(Vb, 0, h), maps[0, h], 128, 64,
                                                1.0 / math.sqrt(cfg.d), M)
        assert (ref[130:256] == 0).all() and (ref[128:130] != 0).any()
        assert (Os[0, 130:, h] == 0).all() and (rms[0, 130:, h] == 0).all()
        assert_close(Os[0, :, h], ref, f"O_s h{h}")


@pytest.mark.parametrize("case", CAUSAL, ids=_id)
def test_causal_lowrank(case):
    cfg, frames, window = case
    say(f"causal low-rank {_id(case)}")
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 3)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    ct, M = _mask(cfg, frames, window)
    Olr, C = sd.sd_lowrank_attn(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), lr, grid=(cfg.T, cfg.Hg, cfg.Wg),
                                block_q=cfg.block_q, chunk_tokens=ct, window=window)
    Olr, C = host(Olr), host(C)
    pos = oracle.token_positions(cfg.T, cfg.Hg, cfg.Wg)
    pairs = oracle.rope_pairs(cfg.rank)
    Pq, Pk = oracle.bf16_bits_to_f64(Pqb), oracle.bf16_bits_to_f64(Pkb)
    n_ar = -(-cfg.L // ct)
    assert C.shape == (cfg.B, cfg.H, n_ar, cfg.rank, cfg.d)
    for b in range(cfg.B):
        for h in range(cfg.H):
            qt = oracle.lowrank_features(_f(Qb, b, h), Pq, pos, pairs)
            kt = oracle.lowrank_features(_f(Kb, b, h), Pk, pos, pairs)
            Cr = oracle.lowrank_states_masked(kt, _f(Vb, b, h), M, ct)
            for c in range(n_ar):
                sc = max(np.abs(Cr[c]).max(), 1e-30)
                assert_close(C[b, h, c] / sc, Cr[c] / sc, f"C[{c}]/max b{b} h{h}", max_abs=1e-4, rel_l2=1e-4)
                s0, e0 = c * ct, min(cfg.L, (c + 1) * ct)
                ref = oracle.lowrank_output(qt[s0:e0], Cr[c], 1e-6)
                assert_close(Olr[b, s0:e0, h], ref, f"O_lr chunk {c} b{b} h{h}")


def _fused_variant(cfg, g, k, select, ct, window, seed=0):
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, seed)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    nq = -(-cfg.L // cfg.block_q)
    idx = torch.empty((cfg.B, cfg.H, nq, k), dtype=torch.int32, device="cuda")
    O = sd.sd_rola_attention(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_f32(g), lr, k,
                             grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q, idx_out=idx, select=select,
                             chunk_tokens=ct if ct < cfg.L else 0, window=window)
    torch.cuda.synchronize()
    return (Qb, Kb, Vb, Pqb, Pkb), host(O), idx.cpu().numpy()


@pytest.mark.parametrize("case", CAUSAL + [(FRAMES, 0, 0), (FRAMES64, 0, 0)], ids=_id)
@pytest.mark.parametrize("select", ["topk", "fixed"])
def test_variant_fused(case, select):
    cfg, frames, window = case
    say(f"fused variant {_id(case)} {select}")
    g = synthetic.gen_gate(cfg, amplified=True)
    k = _kkeep(cfg)
    ct, M = _mask(cfg, frames, window)
    (Qb, Kb, Vb, Pqb, Pkb), O, idx = _fused_variant(cfg, g, k, select, ct, window)
    Pq, Pk = oracle.bf16_bits_to_f64(Pqb), oracle.bf16_bits_to_f64(Pkb)
    allowed = oracle.block_allowed(M, cfg.block_q, cfg.block_k)
    for b in range(cfg.B):
        for h in range(cfg.H):
            Q, K, V = _f(Qb, b, h), _f(Kb, b, h), _f(Vb, b, h)
            res = oracle.rola_attention_head_variant(
                Q, K, V, Q, K, Pq, Pk, g[b].astype(np.float64), T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q,
                bk=cfg.block_k, k_keep=k, sm_scale=1.0 / math.sqrt(cfg.d), select=select,
                chunk_tokens=ct if frames else 0, window=window)
            if select == "fixed":
                assert (idx[b, h] == res["idx"]).all()
            else:
                mism, rows = _map_diff(idx[b, h], res["S"], k, allowed)
                assert mism == 0 and rows == 0, "tie-only differences: compare only unaffected rows"
            assert_close(O[b, :, h], res["O"], f"O b{b} h{h}")


def test_causal_chain_matches_fused():
    # the unfused entry points under the same window give the fused result
    cfg, ct, window = FRAMES, 2 * FRAMES.Hg * FRAMES.Wg, 2
    g = synthetic.gen_gate(cfg, amplified=True)
    k = _kkeep(cfg)
    (Qb, Kb, Vb, Pqb, Pkb), O, idx = _fused_variant(cfg, g, k, "topk", ct, window)
    Q, K, V = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb)
    var = dict(chunk_tokens=ct, window=window)
    idx2 = sd.sd_block_select(Q, K, k, block_q=cfg.block_q, **var)
    assert np.array_equal(idx2.cpu().numpy(), idx)
    Os, _ = sd.sd_sparse_attn(Q, K, V, idx2, block_q=cfg.block_q, **var)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    Olr, _ = sd.sd_lowrank_attn(Q, K, V, lr, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q, **var)
    O2 = sd.sd_gate_fuse(Os, Olr, dev_f32(g))
    assert_close(host(O2), O, "chain vs fused", max_abs=1e-2, rel_l2=1e-3)


def test_causal_720p_sampled():
    # 720P layer as an autoregressive model would run it: chunks of 3 latent
    # frames (10800 tokens), window of 2 chunks; the block map of sampled
    # heads and the output of sampled query blocks around chunk boundaries
    cfg = synthetic.WAN14B_720P
    ct, window = 3 * cfg.Hg * cfg.Wg, 2
    say("causal 720p: generating inputs")
    g = synthetic.gen_gate(cfg, amplified=True)
    k = _kkeep(cfg)
    (Qb, Kb, Vb, Pqb, Pkb), O, idx = _fused_variant(cfg, g, k, "topk", ct, window)
    pos = oracle.token_positions(cfg.T, cfg.Hg, cfg.Wg)
    pairs = oracle.rope_pairs(cfg.rank)
    Pq, Pk = oracle.bf16_bits_to_f64(Pqb), oracle.bf16_bits_to_f64(Pkb)
    nq, nk = -(-cfg.L // cfg.block_q), -(-cfg.L // cfg.block_k)
    # allowed blocks by chunk intervals (the rule the oracle pins against
    # brute force), as the full L x L mask does not fit here
    cq = [((b * 128) // ct, (min(cfg.L, (b + 1) * 128) - 1) // ct) for b in range(nq)]
    ck = [((c * 64) // ct, (min(cfg.L, (c + 1) * 64) - 1) // ct) for c in range(nk)]
    allowed = np.array([[k0 <= q1 and k1 >= q0 - window + 1 for k0, k1 in ck] for q0, q1 in cq])
    scale = 1.0 / math.sqrt(cfg.d)
    blocks = [0, 84, 168, 169, 253, 337, 590]  # chunk starts fall inside blocks 84, 168, 253, 337
    compared = 0
    for h in (0, 27):
        Qh, Kh, Vh = (oracle.bf16_bits_to_f64(x[0, :, h]) for x in (Qb, Kb, Vb))
        S = oracle.block_scores(Qh, Kh, cfg.block_q, cfg.block_k)
        mism, rows = _map_diff(idx[0, h], S, k, allowed)
        say(f"  head {h}: block-map mismatches {mism}, rows with ties {rows}")
        assert mism == 0
        ref_map = oracle.topk_block_map_allowed(S, k, allowed)
        kt = oracle.lowrank_features(Kh, Pk, pos, pairs)
        for qb in blocks:
            if not np.array_equal(idx[0, h, qb], ref_map[qb]):
                continue
            s0, e0 = qb * 128, min(cfg.L, (qb + 1) * 128)
            qi = np.arange(s0, e0)
            Mrows = np.zeros((e0 - s0, cfg.L), dtype=bool)
            for r, i in enumerate(qi):
                c = i // ct
                Mrows[r, max(0, c - window + 1) * ct:min(cfg.L, (c + 1) * ct)] = True
            Os, r_ = oracle.sparse_attention_masked(Qh[s0:e0], Kh, Vh, ref_map[qb:qb + 1], 128, 64, scale, Mrows)
            qt = oracle.lowrank_features(Qh[s0:e0], Pq, pos[s0:e0], pairs)
            Olr = np.empty((e0 - s0, cfg.d))
            for c in sorted(set((qi // ct).tolist())):
                sel = Mrows[(qi // ct).tolist().index(c)]
                Cc = kt[sel].T @ Vh[sel]
                rows_c = qi // ct == c
                Olr[rows_c] = oracle.lowrank_output(qt[rows_c], Cc, 1e-6)
            ref = oracle.gate_fuse(Os, r_, g[0, s0:e0].astype(np.float64), Olr)
            assert_close(O[0, s0:e0, h], ref, f"O head {h} block {qb}")
            compared += 1
    say(f"  compared {compared} query blocks")
    assert compared >= 10
