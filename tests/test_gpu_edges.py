"""Degenerate shapes of the fused layer and the quantiser against the oracle.

robotworld.top SparkDiffusion write-up, section 2.1 (block map, sparse and
low-rank branches, gated fusion) and section 2.3 (per-token FP8 quant):
  * a sequence shorter than one block (21 tokens: one partial query block
    and one partial key block, so every tile is mostly past the end), with
    the backward checked as well;
  * a keep count of 1 on a ragged sequence (each query block keeps its
    single best key block);
  * an empty activation for the quantiser (no rows).
Tolerances are those of the other parity tests (max-abs 2e-2, relative L2
1e-2 for the forward; relative L2 2^-7 for dQ, dK, dV).
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

SUB = synthetic.AttnConfig("sub-block-21", 1, 2, 128, 1, 3, 7, 128, 64, 0.5, 32)
RAGGED = synthetic.AttnConfig("ragged-330", 1, 3, 128, 3, 10, 11, 128, 64, 0.70, 32)
KEEP1 = dataclasses.replace(RAGGED, name="ragged-keep1", sparsity=0.99)


def _run(cfg):
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, 0)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg)
    g = synthetic.gen_gate(cfg, amplified=True)
    k = oracle.keep_count(cfg.sparsity, -(-cfg.L // cfg.block_k))
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    nq = -(-cfg.L // cfg.block_q)
    idx = torch.empty((cfg.B, cfg.H, nq, k), dtype=torch.int32, device="cuda")
    Q, K, V, gd = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_f32(g)
    O = sd.sd_rola_attention(Q, K, V, gd, lr, k, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q, idx_out=idx)
    torch.cuda.synchronize()
    return (Qb, Kb, Vb, Pqb, Pkb, g), (Q, K, V, gd, lr), host(O), idx, k


@pytest.mark.parametrize("cfg", [SUB, KEEP1], ids=lambda c: c.name)
def test_fused_degenerate(cfg):
    say(f"fused {cfg.name}")
    (Qb, Kb, Vb, Pqb, Pkb, g), _, O, idx, k = _run(cfg)
    assert k == 1
    res = oracle.rola_attention(Qb, Kb, Vb, Pqb, Pkb, g, T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q,
                                bk=cfg.block_k, k_keep=k)
    idx = idx.cpu().numpy()
    for (b, h), v in res.items():
        mism, ties, rows = block_map_diff(idx[b, h], v["S"], k)
        assert mism == 0 and rows == 0
        assert_close(O[b, :, h], v["O"], f"O b{b} h{h}")


def test_backward_sub_block():
    cfg = SUB
    say(f"backward {cfg.name}")
    (Qb, Kb, Vb, Pqb, Pkb, g), (Q, K, V, gd, lr), _, idx, k = _run(cfg)
    dOb = synthetic.f32_to_bf16_bits(np.random.default_rng(3).standard_normal(Qb.shape).astype(np.float32))
    grads = sd.sd_rola_backward(Q, K, V, gd, lr, k, idx, dev_bf16(dOb), grid=(cfg.T, cfg.Hg, cfg.Wg),
                                block_q=cfg.block_q)
    torch.cuda.synchronize()
    f = oracle.bf16_bits_to_f64
    idx = idx.cpu().numpy()
    for h in range(cfg.H):
        X = [f(x[0, :, h]) for x in (Qb, Kb, Vb)]
        res = oracle.rola_backward_head(*X, X[0], X[1], f(Pqb), f(Pkb), g[0].astype(np.float64), idx[0, h],
                                        f(dOb[0, :, h]), T=cfg.T, Hg=cfg.Hg, Wg=cfg.Wg, bq=cfg.block_q,
                                        bk=cfg.block_k, sm_scale=1.0 / math.sqrt(cfg.d))
        refs = {"dQ": res["dQ"] + res["dQn"], "dK": res["dK"] + res["dKn"], "dV": res["dV"]}
        for n, r in refs.items():
            got = grads[n][0, :, h].double().cpu().numpy()
            rel = float(np.linalg.norm(got - r) / np.linalg.norm(r))
            say(f"  {n} h{h}: rel_l2={rel:.3e}")
            assert np.isfinite(got).all() and rel <= 2.0 ** -7, (n, h, rel)


def test_quant_no_rows():
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    q, s = sd.sd_quant_fp8_per_token(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 1024) and s.shape == (0,)
