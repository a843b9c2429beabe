"""End-to-end GPU check of the attention block in deployment precision
against the oracle run stage by stage on the same seeded inputs:
x -> FP8 quant + scalar gate -> W8A8 QKV projection -> q/k RMSNorm + 3D
RoPE -> RoLA (block map on Q/K, low-rank branch on the pre-RoPE Qn/Kn,
gated fusion) -> FP8 quant -> W8A8 output projection (robotworld.top
write-up, sections 2.1 and 2.3; kais-engine report, section 2.1).

The oracle stores every tensor that the library passes between kernels in
the same type (bf16 projections, q/k, O; E4M3 codes), rounding its exact
values once. Every stage is checked to its own bar in its own test; here:
  * the block map must be the oracle's except inside a tie window widened
    to what the upstream code differences can do to a score: one-step E4M3
    differences of x and W (below) move the projected q/k by a fraction of
    a percent, so two maps may disagree on blocks whose score lies within
    2^-5 |qbar_b| |kbar_c| of the row's threshold (Cauchy-Schwarz scale of
    the block means, about six times the measured shift); tokens of query
    blocks whose map differs in some head are left out of the output check,
    and at least 3/4 of the tokens must remain;
  * an E4M3 code may land one step (at most 2^-3 of the value) away from
    the oracle's: for x and both weights where x / s lies within 2^-22 of a
    rounding midpoint (the kernel rounds a product, the oracle the
    quotient), and for O also because O reaches its quantiser with the
    attention's own small differences. The output of the last projection is
    then off by at most 2^-3 sum_k |w_nk o_mk| (the oracle's absolute
    products), plus one bf16 rounding, 2^-7 |ref|;
  * overall, rel-L2 <= 2e-2 (the layer's 1e-2 for the attention, doubled
    for the independent FP8 rounding noise of the two sides' O)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from gpu_util import dev_bf16, dev_f32, fp8_code_steps, say
from workloads import synthetic

pytestmark = pytest.mark.gpu


def _b16(x):
    return synthetic.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_deployment_block_tiny_end_to_end():
    cfg = synthetic.AttnConfig("block-small", 1, 4, 128, 4, 16, 16, 128, 64, 0.5, 32)
    L, H, d = cfg.L, cfg.H, cfg.d
    C = H * d
    k_keep = sd.sd_keep_count(cfg.sparsity, L // cfg.block_k)
    x = synthetic.gen_activation(L, C, 21)
    wqkv = synthetic.gen_weight(3 * C, C, 21)
    wo = synthetic.gen_weight(C, C, 22)
    wg = synthetic.gen_gate_weight(C, 21)
    gq, gk = synthetic.gen_norm_weight(C, 21), synthetic.gen_norm_weight(C, 22)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg, 21)
    f = oracle.bf16_bits_to_f64

    # --- oracle, stage by stage
    xq, sx = oracle.quant_fp8_per_token(x)
    g = oracle.gate_gemv(f(x), f(wg), synthetic.GATE_BIAS)
    wq, sw = oracle.quant_weight_per_channel(wqkv)
    y = _b16(oracle.w8a8_gemm(xq, sx, wq, sw))
    pos = oracle.token_positions(cfg.T, cfg.Hg, cfg.Wg)
    Qn, Qr = oracle.qk_norm_rope(f(y[:, :C]), H, d, pos, f(gq))
    Kn, Kr = oracle.qk_norm_rope(f(y[:, C:2 * C]), H, d, pos, f(gk))
    Qn, Qr, Kn, Kr = (_b16(a)[None] for a in (Qn, Qr, Kn, Kr))
    Vb = y[:, 2 * C:].reshape(1, L, H, d)
    res = oracle.rola_attention(Qr, Kr, Vb, Pqb, Pkb, g[None].astype(np.float32), T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg,
                                bq=cfg.block_q, bk=cfg.block_k, k_keep=k_keep, Qnb=Qn, Knb=Kn)
    O = _b16(np.stack([res[(0, h)]["O"] for h in range(H)], axis=1).reshape(L, C))
    oq, so = oracle.quant_fp8_per_token(O)
    woq, swo = oracle.quant_weight_per_channel(wo)
    ref = oracle.w8a8_gemm(oq, so, woq, swo)
    # tie windows of the block map: 2^-5 |qbar_b| |kbar_c| around each row's threshold
    win = []
    for h in range(H):
        qbar = oracle.pooled_means(f(Qr[0, :, h]), cfg.block_q)
        kbar = oracle.pooled_means(f(Kr[0, :, h]), cfg.block_k)
        win.append(2.0 ** -5 * np.outer(np.linalg.norm(qbar, axis=1), np.linalg.norm(kbar, axis=1)))

    # --- library
    X = dev_bf16(x)
    codes, scales, gd = sd.sd_quant_fp8_gate(X, dev_bf16(wg), synthetic.GATE_BIAS)
    Wq, Sw = sd.sd_quant_fp8_per_token(dev_bf16(wqkv))
    Y = sd.sd_gemm_fp8_w8a8(codes, scales, Wq, Sw)
    Q5, K5, Qn5, Kn5, qm5, km5 = sd.sd_qk_norm_rope(Y[:, :C], Y[:, C:2 * C], heads=H, grid=(cfg.T, cfg.Hg, cfg.Wg),
                                                    gamma_q=dev_bf16(gq), gamma_k=dev_bf16(gk), block_means=True,
                                                    block_q=cfg.block_q, block_k=cfg.block_k)
    V5 = Y[:, 2 * C:].unflatten(1, (H, d)).unsqueeze(0)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    ws = sd.rola_workspace(Q5, lr, k_keep, grid=grid, block_q=cfg.block_q)
    idx = torch.empty((1, H, L // cfg.block_q, k_keep), dtype=torch.int32, device="cuda")
    sd.sd_rola_prepare(Q5, K5, V5, lr, k_keep, ws, grid=grid, block_q=cfg.block_q, Qn=Qn5, Kn=Kn5, idx_out=idx,
                       means=(qm5, km5))
    Ob = sd.sd_rola_apply(Q5, K5, V5, gd.view(1, L), lr, k_keep, ws, grid=grid, block_q=cfg.block_q, Qn=Qn5,
                          idx=idx)
    OQ, OS = sd.sd_quant_fp8_per_token(Ob.view(L, C))
    Wo_q, Wo_s = sd.sd_quant_fp8_per_token(dev_bf16(wo))
    out = sd.sd_gemm_fp8_w8a8(OQ, OS, Wo_q, Wo_s)
    torch.cuda.synchronize()

    fp8_code_steps(codes.cpu().numpy(), xq, "x codes")
    fp8_code_steps(Wq.cpu().numpy(), wq, "W_qkv codes")
    fp8_code_steps(Wo_q.cpu().numpy(), woq, "W_out codes")
    got_idx = idx.cpu().numpy()[0]
    nq = L // cfg.block_q
    agree = np.ones(nq, dtype=bool)
    flips = 0
    for h in range(H):
        S, ref_idx = res[(0, h)]["S"], res[(0, h)]["idx"]
        for b in range(nq):
            if np.array_equal(got_idx[h, b], ref_idx[b]):
                continue
            agree[b] = False
            tau = np.sort(S[b])[::-1][k_keep - 1]
            for c in set(got_idx[h, b].tolist()) ^ set(ref_idx[b].tolist()):
                flips += 1
                assert abs(S[b, c] - tau) <= win[h][b, c], f"head {h} row {b}: block {c} outside the tie window"
    tok = np.repeat(agree, cfg.block_q)
    say(f"block map: {flips} blocks differ, all inside the window; {int(tok.sum())} of {L} tokens compared")
    assert tok.mean() >= 0.75
    got = out.float().cpu().numpy().astype(np.float64)[tok]
    ref = ref[tok]
    oq, so = oq[tok], so[tok]
    err = np.abs(got - ref)
    bound = 2.0 ** -3 * oracle.w8a8_abs_products(oq, so, woq, swo) + 2.0 ** -7 * np.abs(ref) + 1e-30
    rel_l2 = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    say(f"block: max |err| {err.max():.3e}, worst err/bound {float((err / bound).max()):.3f}, rel-L2 {rel_l2:.3e}")
    assert float((err / bound).max()) <= 1.0 and rel_l2 <= 2e-2
