"""GPU parity of the RoLA attention path against the CPU oracle.

Every case runs the HIP kernels through the C ABI (via the thin binding) on
seeded inputs and compares element by element with the oracle: the block
map bit-exact outside the tie window, float outputs within max-abs 2e-2 and
relative L2 1e-2. Cases span several tiles, ragged tails (partial query and
key blocks), d = 64 / 128, block_q = 64 / 128, rank 16 / 32, and the
degenerate settings (all blocks kept, zero gate).
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from workloads import synthetic
from gpu_util import assert_close, block_map_diff, dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu

# (name, config) -- small enough for the oracle, several tiles, ragged tails
RAGGED = synthetic.AttnConfig("ragged-330", 1, 3, 128, 3, 10, 11, 128, 64, 0.70, 32)
RAGGED64 = synthetic.AttnConfig("ragged-d64", 2, 2, 64, 5, 7, 13, 64, 64, 0.60, 16)
MID = synthetic.AttnConfig("mid-2176", 1, 4, 128, 2, 32, 34, 128, 64, 0.90, 32)
BQ64 = dataclasses.replace(RAGGED, name="ragged-bq64", block_q=64)
# d = 64 with 128-query blocks: four waves' feature patches share the two
# 8 KB tile buffers, and the rank-16 RoPE split has a pair that starts odd
D64BQ128 = dataclasses.replace(RAGGED64, name="ragged-d64-bq128", block_q=128)
CASES = [synthetic.TINY, RAGGED, RAGGED64, MID, BQ64, D64BQ128]


def _inputs(cfg, seed=0):
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, seed)
    return (Qb, Kb, Vb), tuple(dev_bf16(x) for x in (Qb, Kb, Vb))


def _kkeep(cfg):
    return oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))


def _f(bits, b, h):
    return oracle.bf16_bits_to_f64(bits[b, :, h])


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_block_select(cfg):
    say(f"block_select {cfg.name}")
    (Qb, Kb, _), (Q, K, _) = _inputs(cfg)
    k = _kkeep(cfg)
    idx = sd.sd_block_select(Q, K, k, block_q=cfg.block_q, block_k=cfg.block_k).cpu().numpy()
    tot_ties = 0
    for b in range(cfg.B):
        for h in range(cfg.H):
            S = oracle.block_scores(_f(Qb, b, h), _f(Kb, b, h), cfg.block_q, cfg.block_k)
            mism, ties, _ = block_map_diff(idx[b, h], S, k)
            assert mism == 0, f"(b={b}, h={h}): {mism} blocks differ outside the tie window"
            tot_ties += ties
    say(f"  ties at the threshold: {tot_ties}")


def test_block_select_constructed_ties():
    # every key block has the same mean: all scores of a row are equal, so
    # the map must be the k lowest block indices
    cfg = synthetic.TINY
    rng = np.random.default_rng(0)
    base = synthetic.f32_to_bf16_bits(rng.standard_normal((1, 64, cfg.H, cfg.d)).astype(np.float32))
    Kb = np.tile(base, (1, cfg.L // 64, 1, 1))
    Qb, _, _ = synthetic.gen_qkv(cfg, 1)
    for k in (1, 4, 16):
        idx = sd.sd_block_select(dev_bf16(Qb), dev_bf16(Kb), k, block_q=64, block_k=64).cpu().numpy()
        assert (idx == np.arange(k)[None, None, None, :]).all()


# 140 key blocks: more than 64 blocks can be undecided after the
# approximate scores, which sends a row through the exact in-place path
WIDE = synthetic.AttnConfig("wide-8960", 1, 2, 128, 5, 28, 64, 128, 64, 0.90, 32)


def test_block_select_wide_rows_all_tied():
    # identical key blocks: every score of a row is equal (all 140 blocks
    # undecided), so the map is the k lowest block indices
    cfg = WIDE
    rng = np.random.default_rng(3)
    base = synthetic.f32_to_bf16_bits(rng.standard_normal((1, 64, cfg.H, cfg.d)).astype(np.float32))
    Kb = np.tile(base, (1, cfg.L // 64, 1, 1))
    Qb, _, _ = synthetic.gen_qkv(cfg, 2)
    for k in (1, 10, 70, 140):
        say(f"wide all-tied k={k}")
        idx = sd.sd_block_select(dev_bf16(Qb), dev_bf16(Kb), k, block_q=cfg.block_q, block_k=64).cpu().numpy()
        assert (idx == np.arange(k)[None, None, None, :]).all()


def test_block_select_many_undecided_among_few_candidates():
    # 100 identical key blocks (20..119) score far above the other 40, so a
    # row has about 100 candidates near its k-th score, all of them
    # undecided: more than 64, so the row leaves the compacted path for the
    # full one, whose exact ranking keeps the lowest indices among the ties
    cfg = WIDE
    rng = np.random.default_rng(5)
    u = rng.standard_normal(cfg.d).astype(np.float32)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, cfg.L, cfg.H, cfg.d)).astype(np.float32) + 3.0 * u
    kf = 0.01 * rng.standard_normal((1, cfg.L, cfg.H, cfg.d)).astype(np.float32)
    kf[:, 20 * 64:120 * 64] = 5.0 * u
    Qb, Kb = synthetic.f32_to_bf16_bits(q), synthetic.f32_to_bf16_bits(kf)
    k = 36
    idx = sd.sd_block_select(dev_bf16(Qb), dev_bf16(Kb), k, block_q=cfg.block_q, block_k=64).cpu().numpy()
    assert (idx == np.arange(20, 20 + k)[None, None, None, :]).all()
    for h in range(cfg.H):
        S = oracle.block_scores(_f(Qb, 0, h), _f(Kb, 0, h), cfg.block_q, 64)
        mism, ties, _ = block_map_diff(idx[0, h], S, k)
        say(f"  head {h}: {mism} blocks differ, {ties} ties")
        assert mism == 0


def test_block_select_zero_query_block_and_dominant_key_block():
    # query block 3 is all zeros (its scores are all 0: the k lowest
    # indices); key block 5 is scaled by 2^8, so the largest key-block norm
    # is far above the others and their scores sit near the bottom of the
    # fixed-point range of the approximate scores
    cfg = WIDE
    Qb, Kb, _ = synthetic.gen_qkv(cfg, 4)
    Qb = Qb.copy()
    Kb = Kb.copy()
    Qb[:, 3 * 128:4 * 128] = 0
    kf = oracle.bf16_bits_to_f64(Kb[:, 5 * 64:6 * 64]) * 256.0
    Kb[:, 5 * 64:6 * 64] = synthetic.f32_to_bf16_bits(kf.astype(np.float32))
    k = _kkeep(cfg)
    idx = sd.sd_block_select(dev_bf16(Qb), dev_bf16(Kb), k, block_q=cfg.block_q, block_k=64).cpu().numpy()
    for h in range(cfg.H):
        assert (idx[0, h, 3] == np.arange(k)).all()
        S = oracle.block_scores(_f(Qb, 0, h), _f(Kb, 0, h), cfg.block_q, 64)
        mism, ties, _ = block_map_diff(idx[0, h], S, k)
        say(f"  head {h}: {mism} blocks differ, {ties} ties")
        assert mism == 0


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_sparse_attn(cfg, out_dtype):
    say(f"sparse_attn {cfg.name} {out_dtype}")
    (Qb, Kb, Vb), (Q, K, V) = _inputs(cfg, 1)
    k = _kkeep(cfg)
    scale = 1.0 / math.sqrt(cfg.d)
    maps = np.zeros((cfg.B, cfg.H, -(-cfg.L // cfg.block_q), k), dtype=np.int32)
    for b in range(cfg.B):
        for h in range(cfg.H):
            maps[b, h] = oracle.topk_block_map(oracle.block_scores(_f(Qb, b, h), _f(Kb, b, h), cfg.block_q,
                                                                   cfg.block_k), k)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    Os, rms = sd.sd_sparse_attn(Q, K, V, torch.from_numpy(maps).cuda(), block_q=cfg.block_q, out_dtype=dt)
    Os, rms = host(Os), host(rms)
    for b in range(cfg.B):
        for h in range(cfg.H):
            ref, r = oracle.sparse_attention(_f(Qb, b, h), _f(Kb, b, h), _f(Vb, b, h), maps[b, h], cfg.block_q,
                                             cfg.block_k, scale)
            assert_close(Os[b, :, h], ref, f"O_s b{b} h{h}")
            assert_close(rms[b, :, h], r, f"rms b{b} h{h}")


@pytest.mark.parametrize("cfg", [synthetic.TINY, RAGGED], ids=lambda c: c.name)
def test_sparse_all_blocks_is_dense(cfg):
    (Qb, Kb, Vb), (Q, K, V) = _inputs(cfg, 2)
    nk = -(-cfg.L // cfg.block_k)
    nq = -(-cfg.L // cfg.block_q)
    idx = torch.arange(nk, dtype=torch.int32, device="cuda").expand(cfg.B, cfg.H, nq, nk).contiguous()
    Os, _ = sd.sd_sparse_attn(Q, K, V, idx, block_q=cfg.block_q)
    Os = host(Os)
    for h in range(cfg.H):
        ref = oracle.dense_attention(_f(Qb, 0, h), _f(Kb, 0, h), _f(Vb, 0, h), 1 / math.sqrt(cfg.d))
        assert_close(Os[0, :, h], ref, f"dense h{h}")


def _lowrank_ref(cfg, Qb, Kb, Vb, Pqb, Pkb, b, h):
    pos = oracle.token_positions(cfg.T, cfg.Hg, cfg.Wg)
    pairs = oracle.rope_pairs(cfg.rank)
    Pq, Pk = oracle.bf16_bits_to_f64(Pqb), oracle.bf16_bits_to_f64(Pkb)
    qt = oracle.lowrank_features(_f(Qb, b, h), Pq, pos, pairs)
    kt = oracle.lowrank_features(_f(Kb, b, h), Pk, pos, pairs)
    C = oracle.lowrank_state(kt, _f(Vb, b, h))
    return C, oracle.lowrank_output(qt, C, 1e-6)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_lowrank(cfg):
    say(f"lowrank {cfg.name}")
    (Qb, Kb, Vb), (Q, K, V) = _inputs(cfg, 3)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    Olr, C = sd.sd_lowrank_attn(Q, K, V, lr, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q)
    Olr, C = host(Olr), host(C)
    for b in range(cfg.B):
        for h in range(cfg.H):
            Cr, Or = _lowrank_ref(cfg, Qb, Kb, Vb, Pqb, Pkb, b, h)
            scale = np.abs(Cr).max()
            assert_close(C[b, h] / scale, Cr / scale, f"C/max|C| b{b} h{h}", max_abs=1e-4, rel_l2=1e-4)
            assert_close(Olr[b, :, h], Or, f"O_lr b{b} h{h}")


def _close_bf16_out(got, ref, name):
    # O is stored as bf16: allow its rounding (half an ulp, 2^-9 relative)
    # on top of the accuracy bound of the f32 result
    err = np.abs(got - ref)
    bound = 2e-2 + 2.0 ** -9 * np.abs(ref)
    say(f"  {name}: max_abs={err.max():.3e} worst err/bound={(err / bound).max():.3f}")
    assert (err <= bound).all(), name
    assert_close(got, ref, name, max_abs=np.inf)


def test_gate_fuse():
    # O_s at the scale of attention outputs, O_lr of unit RMS, gates N(1, 1)
    cfg = RAGGED
    rng = np.random.default_rng(4)
    Os = (0.5 * rng.standard_normal((1, cfg.L, cfg.H, cfg.d))).astype(np.float32)
    Olr = rng.standard_normal((1, cfg.L, cfg.H, cfg.d)).astype(np.float32)
    g = synthetic.gen_gate(cfg, amplified=True)
    O = host(sd.sd_gate_fuse(dev_f32(Os), dev_f32(Olr), dev_f32(g)))
    for h in range(cfg.H):
        os_, ol = Os[0, :, h].astype(np.float64), Olr[0, :, h].astype(np.float64)
        r = np.sqrt((os_ ** 2).mean(axis=1))
        _close_bf16_out(O[0, :, h], oracle.gate_fuse(os_, r, g[0].astype(np.float64), ol), f"O h{h}")
    # per-(token, head) gates
    g3 = rng.standard_normal((1, cfg.L, cfg.H)).astype(np.float32)
    O3 = host(sd.sd_gate_fuse(dev_f32(Os), dev_f32(Olr), dev_f32(g3)))
    for h in range(cfg.H):
        os_, ol = Os[0, :, h].astype(np.float64), Olr[0, :, h].astype(np.float64)
        r = np.sqrt((os_ ** 2).mean(axis=1))
        _close_bf16_out(O3[0, :, h], oracle.gate_fuse(os_, r, g3[0, :, h].astype(np.float64), ol), f"O3 h{h}")
    # bf16 inputs
    Ob = host(sd.sd_gate_fuse(dev_f32(Os).bfloat16(), dev_f32(Olr).bfloat16(), dev_f32(g)))
    for h in range(cfg.H):
        osb = host(dev_f32(Os[0, :, h]).bfloat16())
        olb = host(dev_f32(Olr[0, :, h]).bfloat16())
        r = np.sqrt((osb ** 2).mean(axis=1))
        _close_bf16_out(Ob[0, :, h], oracle.gate_fuse(osb, r, g[0].astype(np.float64), olb), f"O bf16-in h{h}")


def _fused(cfg, gate, seed=0, Qn=None, Kn=None):
    (Qb, Kb, Vb), (Q, K, V) = _inputs(cfg, seed)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    k = _kkeep(cfg)
    nq = -(-cfg.L // cfg.block_q)
    idx = torch.empty((cfg.B, cfg.H, nq, k), dtype=torch.int32, device="cuda")
    O = sd.sd_rola_attention(Q, K, V, dev_f32(gate), lr, k, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q,
                             idx_out=idx, Qn=Qn, Kn=Kn)
    torch.cuda.synchronize()
    return (Qb, Kb, Vb, Pqb, Pkb), O, idx.cpu().numpy(), k


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("amplified", [False, True], ids=["gate", "gate-amplified"])
def test_rola_fused(cfg, amplified):
    say(f"rola fused {cfg.name} amplified={amplified}")
    g = synthetic.gen_gate(cfg, amplified=amplified)
    (Qb, Kb, Vb, Pqb, Pkb), O, idx, k = _fused(cfg, g)
    O = host(O)
    res = oracle.rola_attention(Qb, Kb, Vb, Pqb, Pkb, g, T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q,
                                bk=cfg.block_k, k_keep=k)
    for (b, h), v in res.items():
        mism, ties, rows = block_map_diff(idx[b, h], v["S"], k)
        assert mism == 0
        assert rows == 0, "tie-only differences: compare only unaffected rows"
        assert_close(O[b, :, h], v["O"], f"O b{b} h{h}")


def test_rola_zero_gate_is_sparse_branch_bitwise():
    cfg = RAGGED
    g = np.zeros((cfg.B, cfg.L), dtype=np.float32)
    (Qb, Kb, Vb, _, _), O, idx, k = _fused(cfg, g)
    Q, K, V = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb)
    Os, _ = sd.sd_sparse_attn(Q, K, V, torch.from_numpy(idx).cuda(), block_q=cfg.block_q, out_dtype=torch.bfloat16)
    assert torch.equal(O.view(torch.int16), Os.view(torch.int16))


def test_rola_separate_normalised_qk():
    # the low-rank branch reads Qn / Kn when given (pre-RoPE normalised q/k)
    cfg = RAGGED
    g = synthetic.gen_gate(cfg, amplified=True)
    Qnb, Knb, _ = synthetic.gen_qkv(cfg, 11)
    (Qb, Kb, Vb, Pqb, Pkb), O, idx, k = _fused(cfg, g, Qn=dev_bf16(Qnb), Kn=dev_bf16(Knb))
    res = oracle.rola_attention(Qb, Kb, Vb, Pqb, Pkb, g, T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q,
                                bk=cfg.block_k, k_keep=k, Qnb=Qnb, Knb=Knb)
    O = host(O)
    for (b, h), v in res.items():
        assert_close(O[b, :, h], v["O"], f"O(Qn,Kn) h{h}")


@pytest.mark.parametrize("cfg", [RAGGED, RAGGED64], ids=lambda c: c.name)
def test_rola_per_head_projections(cfg):
    # one P_q and P_k per head (P_head_stride = rank * d)
    say(f"rola fused {cfg.name}, per-head projections")
    g = synthetic.gen_gate(cfg, amplified=True)
    (Qb, Kb, Vb), (Q, K, V) = _inputs(cfg, 2)
    pp = [synthetic.gen_lowrank_params(cfg, seed=11 + h) for h in range(cfg.H)]
    Pqb, Pkb = np.stack([x[0] for x in pp]), np.stack([x[1] for x in pp])
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb), head_stride=cfg.rank * cfg.d)
    k = _kkeep(cfg)
    nq = -(-cfg.L // cfg.block_q)
    idx = torch.empty((cfg.B, cfg.H, nq, k), dtype=torch.int32, device="cuda")
    O = sd.sd_rola_attention(Q, K, V, dev_f32(g), lr, k, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q,
                             idx_out=idx)
    torch.cuda.synchronize()
    O, idx = host(O), idx.cpu().numpy()
    f = oracle.bf16_bits_to_f64
    for b in range(cfg.B):
        for h in range(cfg.H):
            X = [f(x[b, :, h]) for x in (Qb, Kb, Vb)]
            v = oracle.rola_attention_head(*X, X[0], X[1], f(Pqb[h]), f(Pkb[h]), np.asarray(g[b], dtype=np.float64),
                                           T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q, bk=cfg.block_k, k_keep=k,
                                           sm_scale=1.0 / math.sqrt(cfg.d))
            mism, ties, rows = block_map_diff(idx[b, h], v["S"], k)
            assert mism == 0 and rows == 0
            assert_close(O[b, :, h], v["O"], f"O b{b} h{h}")


def test_rola_deterministic():
    cfg = MID
    g = synthetic.gen_gate(cfg, amplified=True)
    _, O1, i1, _ = _fused(cfg, g)
    _, O2, i2, _ = _fused(cfg, g)
    assert np.array_equal(i1, i2)
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))


def test_chain_matches_fused():
    # the unfused entry points composed give the fused result
    cfg = MID
    g = synthetic.gen_gate(cfg, amplified=True)
    (Qb, Kb, Vb, Pqb, Pkb), O, idx, k = _fused(cfg, g)
    Q, K, V = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb)
    idx2 = sd.sd_block_select(Q, K, k, block_q=cfg.block_q)
    assert np.array_equal(idx2.cpu().numpy(), idx)
    Os, _ = sd.sd_sparse_attn(Q, K, V, idx2, block_q=cfg.block_q)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    Olr, _ = sd.sd_lowrank_attn(Q, K, V, lr, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q)
    O2 = sd.sd_gate_fuse(Os, Olr, dev_f32(g))
    assert_close(host(O2), host(O), "chain vs fused", max_abs=1e-2, rel_l2=1e-3)
