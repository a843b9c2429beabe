"""GPU parity of the W8A8 FP8 projection (sd_gemm_fp8_w8a8) against the
oracle's float64 product of the dequantised operands.

Acceptance per element (derived from the arithmetic): the kernel rounds the
f32 accumulator times the two scales once to bf16: at most one bf16 ulp,
2^-7 |y_ref|, once the accumulator carries its own error (the rounding can
land on the other neighbour). The accumulator is a sum of 64-product MFMA
blocks. The matrix unit adds the exact E4M3 products of each group of 8 with
about 13 bits below the group's largest magnitude (measured on the hardware: a
term 2^-12 below the largest survives, one 2^-14 below is dropped), so a
group loses at most 7 * 2^-13 of its largest term; with margin the bound
takes 2^-9 sum_k |terms|, plus 2^-126 for underflow."""
import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from gpu_util import dev_bf16, say
from workloads import synthetic

pytestmark = pytest.mark.gpu


def _bound(xq, sx, wq, sw, ref, K):
    absp = oracle.w8a8_abs_products(xq, sx, wq, sw)
    return 2.0 ** -7 * np.abs(ref) + 2.0 ** -9 * absp + 2.0 ** -126


def _check(y, ref, bound, name):
    y = np.asarray(y, dtype=np.float64)
    assert np.isfinite(y).all(), name
    err = np.abs(y - ref)
    worst = float((err / bound).max())
    say(f"{name}: max |err| {err.max():.3e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0, name


def _host_bf16(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (300, 198, 128), (1000, 384, 512), (37, 520, 5120)])
def test_gemm_quantised_activation_and_weight(M, N, K):
    say(f"case M={M} N={N} K={K}")
    xb = synthetic.gen_activation(M, K, seed=M)
    wb = synthetic.gen_weight(N, K, seed=N)
    xq, sx = oracle.quant_fp8_per_token(xb)
    wq, sw = oracle.quant_weight_per_channel(wb)
    ref = oracle.w8a8_gemm(xq, sx, wq, sw)
    ldy = (N + 3) // 4 * 4
    out = torch.full((M, ldy), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :N]
    y = sd.sd_gemm_fp8_w8a8(torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(wq).cuda(),
                            torch.from_numpy(sw).cuda(), out=out)
    torch.cuda.synchronize()
    _check(_host_bf16(y), ref, _bound(xq, sx, wq, sw, ref, K), f"gemm {M}x{N}x{K}")


def test_gemm_strided_operands():
    M, N, K = 200, 136, 192
    xq, sx = synthetic.gen_fp8_codes(M, K, seed=1)
    wq, sw = synthetic.gen_fp8_codes(N, K, seed=2)
    ref = oracle.w8a8_gemm(xq, sx, wq, sw)
    xbig = torch.zeros((M, K + 64), dtype=torch.uint8)
    xbig[:, 16:16 + K] = torch.from_numpy(xq)
    wbig = torch.zeros((N, K + 32), dtype=torch.uint8)
    wbig[:, :K] = torch.from_numpy(wq)
    xd, wd = xbig.cuda()[:, 16:16 + K], wbig.cuda()[:, :K]
    outbig = torch.zeros((M, N + 8), dtype=torch.bfloat16, device="cuda")
    y = sd.sd_gemm_fp8_w8a8(xd, torch.from_numpy(sx).cuda(), wd, torch.from_numpy(sw).cuda(), out=outbig[:, :N])
    torch.cuda.synchronize()
    _check(_host_bf16(y), ref, _bound(xq, sx, wq, sw, ref, K), "gemm strided")
    assert float(outbig[:, N:].float().abs().max()) == 0.0  # nothing written past N


def test_gemm_integer_operands_exact():
    # small integer codes with unit scales: products are integers <= 16 and
    # within 8 bits of each other, so every partial sum is exact and the
    # result is exact up to the bf16 rounding
    rng = np.random.default_rng(5)
    M, N, K = 64, 96, 256
    table = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4, 0xC8], dtype=np.uint8)
    xq = table[rng.integers(0, 9, (M, K))]
    wq = table[rng.integers(0, 9, (N, K))]
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    ref = oracle.w8a8_gemm(xq, ones_m, wq, ones_n)
    y = sd.sd_gemm_fp8_w8a8(torch.from_numpy(xq).cuda(), torch.from_numpy(ones_m).cuda(),
                            torch.from_numpy(wq).cuda(), torch.from_numpy(ones_n).cuda())
    torch.cuda.synchronize()
    got = _host_bf16(y)
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()  # RNE of exact integers
    assert np.array_equal(got, ref_bf16)


def test_gemm_720p_qkv_sampled_rows():
    # the QKV projection of the 720P block at full size (75600 x 15360 x
    # 5120) on random finite codes; rows sampled across every tile row,
    # all columns checked
    M, N, K = synthetic.PROJ_QKV_720P
    xq, sx = synthetic.gen_fp8_codes(M, K, seed=11)
    wq, sw = synthetic.gen_fp8_codes(N, K, seed=12)
    y = sd.sd_gemm_fp8_w8a8(torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(wq).cuda(),
                            torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 4999), [M - 1, M - 80, 255, 256]]))
    got = _host_bf16(y[torch.from_numpy(rows).cuda()])
    ref = oracle.w8a8_gemm(xq[rows], sx[rows], wq, sw)
    _check(got, ref, _bound(xq[rows], sx[rows], wq, sw, ref, K), "gemm 720p qkv sampled")


def test_gemm_deterministic():
    M, N, K = 512, 512, 1024
    xq, sx = synthetic.gen_fp8_codes(M, K, seed=3)
    wq, sw = synthetic.gen_fp8_codes(N, K, seed=4)
    args = [torch.from_numpy(a).cuda() for a in (xq, sx, wq, sw)]
    y1 = sd.sd_gemm_fp8_w8a8(*args)
    y2 = sd.sd_gemm_fp8_w8a8(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
