"""GPU parity of the q/k producer (sd_qk_norm_rope: RMSNorm of each
projection row, then the backbone 3D RoPE per head) against the oracle's
float64 values.

Acceptance per element (derived from the arithmetic): the kernel computes
in f32 and rounds once to bf16, so it is within one bf16 ulp of the exact
value, 2^-7 |ref|, once its f32 error is counted (the rounding can land on
the other neighbour). The f32 error of a rotated channel is dominated by the
angle p*theta formed in f32 (|p| <= 80: 80 * 2^-24 rad) and by cancellation
in u cos - v sin, both at most about 2^-18 (|u| + |v|) of the pair's
unrotated values; the bound takes 2^-16 (|u| + |v|) with margin. For the
unrotated output the second term is 2^-20 |ref| (the f32 sum of squares
over at most 8192 channels)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from gpu_util import dev_bf16, say
from workloads import synthetic

pytestmark = pytest.mark.gpu


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


def _pair_mag(Xn):
    # |u| + |v| of the pair each channel belongs to (pairs (2m, 2m+1))
    a = np.abs(Xn)
    s = a[..., 0::2] + a[..., 1::2]
    return np.repeat(s, 2, axis=-1)


def _check(name, got, ref, extra):
    err = np.abs(got - ref)
    bound = 2.0 ** -7 * np.abs(ref) + extra + 2.0 ** -126
    worst = float((err / bound).max())
    say(f"{name}: max |err| {err.max():.3e}, worst err/bound {worst:.3f}")
    assert np.isfinite(got).all() and worst <= 1.0, name


def _run_case(B, T, Hg, Wg, H, d, seed, strided=False, with_gamma=True, block_q=0):
    L = T * Hg * Wg
    C = H * d
    qb = synthetic.gen_qk_rows(B * L, C, seed)
    kb = synthetic.gen_qk_rows(B * L, C, seed + 1)
    gq = synthetic.gen_norm_weight(C, seed) if with_gamma else None
    gk = synthetic.gen_norm_weight(C, seed + 1) if with_gamma else None
    if strided:  # q and k as slices of one [rows, 3C] projection output
        buf = np.zeros((B * L, 3 * C), dtype=np.uint16)
        buf[:, :C], buf[:, C:2 * C] = qb, kb
        dbuf = dev_bf16(buf)
        q, k = dbuf[:, :C], dbuf[:, C:2 * C]
    else:
        q, k = dev_bf16(qb), dev_bf16(kb)
    res = sd.sd_qk_norm_rope(q, k, heads=H, grid=(T, Hg, Wg), batch=B,
                             gamma_q=dev_bf16(gq) if with_gamma else None,
                             gamma_k=dev_bf16(gk) if with_gamma else None,
                             block_means=block_q > 0, block_q=block_q or 128, block_k=64)
    Q, K, Qn, Kn = res[:4]
    torch.cuda.synchronize()
    pos = oracle.token_positions(T, Hg, Wg)
    for name, xb, g, outr, outn in (("q", qb, gq, Q, Qn), ("k", kb, gk, K, Kn)):
        gam = oracle.bf16_bits_to_f64(g) if g is not None else None
        for b in range(B):
            X = oracle.bf16_bits_to_f64(xb[b * L:(b + 1) * L])
            Xn, Xr = oracle.qk_norm_rope(X, H, d, pos, gam, 1e-6)
            _check(f"{name}n b{b}", _f(outn[b]), Xn, 2.0 ** -20 * np.abs(Xn))
            _check(f"{name} rope b{b}", _f(outr[b]), Xr, 2.0 ** -16 * _pair_mag(Xn))
    if block_q:
        # the block means of the stored rotated outputs, exact in float64
        qm, km = (m.cpu().numpy() for m in res[4:])
        for b in range(B):
            for h in range(H):
                assert np.array_equal(qm[b, h], oracle.pooled_means(_f(Q[b, :, h]), block_q)), (b, h)
                assert np.array_equal(km[b, h], oracle.pooled_means(_f(K[b, :, h]), 64)), (b, h)


@pytest.mark.parametrize("B,T,Hg,Wg,H", [(1, 3, 5, 7, 4), (2, 2, 4, 9, 12), (1, 4, 6, 10, 40)])
def test_qk_norm_rope_small(B, T, Hg, Wg, H):
    say(f"case B={B} grid={T}x{Hg}x{Wg} H={H}")
    _run_case(B, T, Hg, Wg, H, 128, seed=B * 100 + H)


def test_qk_norm_rope_strided_rows_no_gamma():
    _run_case(1, 3, 4, 5, 8, 128, seed=9, strided=True, with_gamma=False)


def test_qk_norm_rope_720p_sampled_rows():
    # 75600 tokens x 40 heads x 128: q and k at full size, rows sampled
    # across the sequence (all heads and channels of each sampled row)
    T, Hg, Wg, H, d = 21, 45, 80, 40, 128
    L, C = T * Hg * Wg, H * d
    qb = synthetic.gen_qk_rows(L, C, 31)
    kb = synthetic.gen_qk_rows(L, C, 32)
    gq, gk = synthetic.gen_norm_weight(C, 31), synthetic.gen_norm_weight(C, 32)
    Q, K, Qn, Kn = sd.sd_qk_norm_rope(dev_bf16(qb), dev_bf16(kb), heads=H, grid=(T, Hg, Wg),
                                      gamma_q=dev_bf16(gq), gamma_k=dev_bf16(gk))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, L, 997), [L - 1, 3599, 3600, 79, 80]]))
    pos = oracle.token_positions(T, Hg, Wg)[rows]
    ridx = torch.from_numpy(rows).cuda()
    for name, xb, g, outr, outn in (("q", qb, gq, Q, Qn), ("k", kb, gk, K, Kn)):
        Xn, Xr = oracle.qk_norm_rope(oracle.bf16_bits_to_f64(xb[rows]), H, d, pos, oracle.bf16_bits_to_f64(g))
        _check(f"{name}n 720p", _f(outn[0][ridx]), Xn, 2.0 ** -20 * np.abs(Xn))
        _check(f"{name} rope 720p", _f(outr[0][ridx]), Xr, 2.0 ** -16 * _pair_mag(Xn))


def test_qk_norm_rope_deterministic():
    qb = synthetic.gen_qk_rows(2 * 60, 1024, 5)
    q = dev_bf16(qb)
    a = sd.sd_qk_norm_rope(q, q, heads=8, grid=(3, 4, 5), batch=2)
    b = sd.sd_qk_norm_rope(q, q, heads=8, grid=(3, 4, 5), batch=2)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # q and k from the same rows give the same outputs
    assert torch.equal(a[0].view(torch.int16), a[1].view(torch.int16))


# --- block means of the rotated outputs --------------------------------------
# The producer's q-bar / k-bar are float64 sums of the stored bf16 values in
# token order divided by the block's token count. For these inputs the sums
# are exact in float64 (a block's values span far fewer than 38 binades), so
# they must equal the oracle's means of the produced Q / K bit for bit,
# whatever the summation order.

@pytest.mark.parametrize("B,T,Hg,Wg,H,bq", [(2, 3, 5, 7, 4, 128), (1, 5, 9, 11, 3, 64), (1, 4, 16, 16, 40, 128)])
def test_qk_norm_rope_block_means(B, T, Hg, Wg, H, bq):
    # the producer with block means: its outputs against the oracle as
    # above, its means against the oracle's means of those outputs
    say(f"block means B={B} grid={T}x{Hg}x{Wg} H={H} block_q={bq}")
    _run_case(B, T, Hg, Wg, H, 128, seed=B * 10 + H, block_q=bq)


def test_prepare_with_producer_means_equals_pooling():
    # the block map and the fused output from the producer's means equal
    # those of the prepare phase pooling Q and K itself
    cfg = synthetic.AttnConfig("producer-means", 1, 4, 128, 4, 16, 16, 128, 64, 0.75, 32)
    C = cfg.H * cfg.d
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    q = dev_bf16(synthetic.gen_qk_rows(cfg.L, C, 21))
    k = dev_bf16(synthetic.gen_qk_rows(cfg.L, C, 22))
    v = dev_bf16(synthetic.gen_qk_rows(cfg.L, C, 23)).view(1, cfg.L, cfg.H, cfg.d)
    Q, K, Qn, Kn, qm, km = sd.sd_qk_norm_rope(q, k, heads=cfg.H, grid=grid, block_means=True)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    k_keep = oracle.keep_count(cfg.sparsity, cfg.L // 64)
    g = torch.ones((1, cfg.L), dtype=torch.float32, device="cuda")
    outs = []
    for means in (None, (qm, km)):
        ws = sd.rola_workspace(Q, lr, k_keep, grid=grid)
        idx = torch.empty((1, cfg.H, cfg.L // 128, k_keep), dtype=torch.int32, device="cuda")
        sd.sd_rola_prepare(Q, K, v, lr, k_keep, ws, grid=grid, Qn=Qn, Kn=Kn, idx_out=idx, means=means)
        O = sd.sd_rola_apply(Q, K, v, g, lr, k_keep, ws, grid=grid, Qn=Qn, idx=idx)
        torch.cuda.synchronize()
        outs.append((idx.cpu(), O.view(torch.int16).cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_qk_norm_rope_block_means_720p_sampled_blocks():
    # full 720P size (75600 tokens, 40 heads): the means of sampled query
    # and key blocks, including the partial tails, against the oracle's means
    # of the produced Q / K rows of those blocks
    T, Hg, Wg, H, d = 21, 45, 80, 40, 128
    L, C = T * Hg * Wg, H * d
    q = dev_bf16(synthetic.gen_qk_rows(L, C, 41))
    k = dev_bf16(synthetic.gen_qk_rows(L, C, 42))
    Q, K, Qn, Kn, qm, km = sd.sd_qk_norm_rope(q, k, heads=H, grid=(T, Hg, Wg), block_means=True)
    torch.cuda.synchronize()
    qm, km = qm.cpu().numpy(), km.cpu().numpy()
    for X, M, bs, blocks in ((Q, qm, 128, [0, 1, 295, 590]), (K, km, 64, [0, 1, 590, 1181])):
        for c in blocks:
            rows = _f(X[0, c * bs:min(L, (c + 1) * bs)])  # [tokens, H, d]
            ref = rows.sum(axis=0) / rows.shape[0]
            assert np.array_equal(M[0, :, c], ref), (bs, c)
    say("720P block means: sampled query and key blocks exact")
