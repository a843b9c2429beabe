"""GPU parity of the per-token FP8 E4M3 quantiser against the oracle.

The oracle's code is the definition, E4M3(x / s) for the stored scale s
(robotworld.top write-up, section 2.3: per-token dynamic scale). The kernel
rounds x * fp32(448 / amax), which lies within 2^-22 of x / s, so a code
may land one step away where x / s is that close to a rounding midpoint:
codes must be within one step (the sign-magnitude code index), and the
number that differ is printed. Scales are one correctly rounded f32
division on both sides and must match bit for bit. Where the scale is
exactly 1 (|x|max = 448) the product is x itself and the codes must match
bit for bit too.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_rank_attention_rola_amd as sd
from workloads import synthetic
from gpu_util import dev_bf16, fp8_code_steps, say

pytestmark = pytest.mark.gpu


def _run(x_bits):
    q, s = sd.sd_quant_fp8_per_token(dev_bf16(x_bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1001, 5120), (37, 1024), (5, 136), (3, 8), (64, 16384)])
def test_quant_random_rows(M, K):
    say(f"quant M={M} K={K}")
    x = synthetic.gen_activation(M, K, seed=M + K)
    q, s = _run(x)
    q_ref, s_ref = oracle.quant_fp8_per_token(x)
    assert np.array_equal(s, s_ref)
    fp8_code_steps(q, q_ref, f"{M}x{K}")


def _bf16_bits(v):
    return synthetic.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_quant_codec_edges_through_kernel():
    # Rows whose |x|max is 448 have a scale of exactly 1, so every value is
    # converted as is: all E4M3 values, all midpoints between neighbours
    # (ties to even), values just off the midpoints and tiny values.
    vals = oracle.e4m3_decode(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -100]])
    bits = _bf16_bits(pts)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), pts.astype(np.float32).astype(np.float64))
    mb = _bf16_bits(mids[1:])
    bits = np.concatenate([bits, mb + 1, mb - 1])  # one bf16 step either side of each midpoint
    bits = np.concatenate([bits, bits | 0x8000])
    K = 512
    row = np.zeros(K, dtype=np.uint16)
    n = len(bits)
    rows = []
    for s0 in range(0, n, K - 8):
        r = row.copy()
        chunk = bits[s0:s0 + K - 8]
        r[:len(chunk)] = chunk
        r[K - 1] = _bf16_bits([448.0])[0]
        rows.append(r)
    x = np.stack(rows)
    q, s = _run(x)
    q_ref, s_ref = oracle.quant_fp8_per_token(x)
    assert (s == np.float32(1.0)).all()
    assert np.array_equal(s, s_ref)
    assert np.array_equal(q, q_ref)


def test_quant_zero_and_constant_rows():
    x = np.zeros((6, 64), dtype=np.uint16)
    x[1] = _bf16_bits([-3.5])[0]
    x[2, ::2] = _bf16_bits([1e-20])[0]
    x[3, 5] = _bf16_bits([1e30])[0]
    x[4] = _bf16_bits(np.linspace(-2, 2, 64))
    q, s = _run(x)
    q_ref, s_ref = oracle.quant_fp8_per_token(x)
    assert np.array_equal(s, s_ref)
    fp8_code_steps(q, q_ref, "zero and constant rows")


def test_quant_strided_rows():
    M, K, ld = 40, 256, 320
    x = synthetic.gen_activation(M, ld, seed=9)
    xd = dev_bf16(x)[:, :K]
    qbuf = torch.full((M, 264), 0xAA, dtype=torch.uint8, device="cuda")
    q, s = sd.sd_quant_fp8_per_token(xd, q=qbuf[:, :K])
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_fp8_per_token(x[:, :K])
    fp8_code_steps(qbuf[:, :K].cpu().numpy(), q_ref, "strided rows")
    assert (qbuf[:, K:].cpu().numpy() == 0xAA).all()  # nothing written past K
    assert np.array_equal(s.cpu().numpy(), s_ref)


def test_quant_480p_activation_sampled_rows():
    M, K = synthetic.QUANT_480P
    say(f"quant full size {M}x{K}")
    x = synthetic.gen_activation(M, K, seed=0)
    q, s = _run(x)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 1024, replace=False)]))
    q_ref, s_ref = oracle.quant_fp8_per_token(x[rows])
    assert np.array_equal(s[rows], s_ref)
    fp8_code_steps(q[rows], q_ref, f"480P activation, {len(rows)} sampled rows")
    # every row's largest-magnitude element lands on +-448 (0x7E / 0xFE)
    xf = oracle.bf16_bits_to_f64(x[rows])
    arg = np.abs(xf).argmax(axis=1)
    assert ((q[rows][np.arange(len(rows)), arg] & 0x7F) == 0x7E).all()


def test_quant_720p_activation_sampled_rows():
    M, K = synthetic.QUANT_720P
    say(f"quant full size {M}x{K}")
    x = synthetic.gen_activation(M, K, seed=5)
    q, s = _run(x)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    q_ref, s_ref = oracle.quant_fp8_per_token(x[rows])
    assert np.array_equal(s[rows], s_ref)
    fp8_code_steps(q[rows], q_ref, f"720P activation, {len(rows)} sampled rows")


def test_quant_rows_with_exact_ties():
    # |x|max with a bf16 significand that is a multiple of 7: x / s then
    # lands exactly on rounding midpoints for many x, where the kernel's
    # product may round either way; every such code must still be within
    # one step, and every code of a row with a power-of-two scale exact.
    x = synthetic.gen_activation(16, 4096, seed=31)
    xf = oracle.bf16_bits_to_f64(x).astype(np.float32)
    for i, b in enumerate([140, 168, 196, 210, 252, 154, 182, 224]):
        amax = np.float32(b) * np.float32(2.0 ** -5)
        xf[i] = np.clip(xf[i], -0.99 * amax, 0.99 * amax)
        xf[i, np.abs(xf[i]).argmax()] = amax
    x = synthetic.f32_to_bf16_bits(xf)
    q, s = _run(x)
    q_ref, s_ref = oracle.quant_fp8_per_token(x)
    assert np.array_equal(s, s_ref)
    fp8_code_steps(q, q_ref, "rows with exact ties")
    # 224 / 448 = 1/2: the scale is a power of two and the product exact
    assert np.array_equal(q[7], q_ref[7])


# --- the quantiser with the scalar gate folded in ----------------------------
# Codes and scales must equal the plain quantiser's bit for bit. The gate is
# an f32 sum of K products: each lane adds its 8*VPL <= 80 terms in order,
# then a 6-level tree adds the 64 lane sums and the bias is added once, so
# |g - ref| <= 88 * 2^-24 * sum |w x| + 2^-24 |ref| (f32 rounding of each
# step); the test takes 2^-17 sum |w x| + 2^-23 |ref|.

def _gate_bound(xb, wb, ref):
    absx = oracle.bf16_bits_to_f64(xb)
    absw = oracle.bf16_bits_to_f64(wb)
    return 2.0 ** -17 * oracle.gate_abs_terms(absx, absw) + 2.0 ** -23 * np.abs(ref) + 1e-30


@pytest.mark.parametrize("M,K", [(1000, 5120), (37, 1024), (5, 136), (64, 16384)])
def test_quant_gate_matches_quant_and_oracle(M, K):
    say(f"quant+gate M={M} K={K}")
    x = synthetic.gen_activation(M, K, seed=M + 3 * K)
    w = synthetic.gen_gate_weight(K, seed=K)
    xd = dev_bf16(x)
    q, s, g = sd.sd_quant_fp8_gate(xd, dev_bf16(w), synthetic.GATE_BIAS)
    q0, s0 = sd.sd_quant_fp8_per_token(xd)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32))
    ref = oracle.gate_gemv(oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(w), synthetic.GATE_BIAS)
    got = g.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    worst = float((err / _gate_bound(x, w, ref)).max())
    say(f"gate: max |err| {err.max():.3e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0


def test_quant_gate_720p_full_rows_sampled():
    M, K = synthetic.QUANT_720P
    x = synthetic.gen_activation(M, K, seed=77)
    w = synthetic.gen_gate_weight(K, seed=77)
    xd = dev_bf16(x)
    q, s, g = sd.sd_quant_fp8_gate(xd, dev_bf16(w), synthetic.GATE_BIAS)
    q0, s0 = sd.sd_quant_fp8_per_token(xd)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32))
    rows = np.unique(np.concatenate([np.arange(0, M, 331), [M - 1]]))
    ref = oracle.gate_gemv(oracle.bf16_bits_to_f64(x[rows]), oracle.bf16_bits_to_f64(w), synthetic.GATE_BIAS)
    got = g.cpu().numpy().astype(np.float64)[rows]
    worst = float((np.abs(got - ref) / _gate_bound(x[rows], w, ref)).max())
    say(f"gate 720p: worst err/bound {worst:.3f}")
    assert worst <= 1.0
