"""Pins of the W8A8 FP8 projection oracle (oracle/gemm.py) against brute
force, integer arithmetic and exact scaling identities."""
import numpy as np
import pytest

import oracle

# E4M3FN codes of the integers -4..4 (OCP 8-bit FP spec: bias 7, 3 mantissa bits)
INT_CODES = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, -1: 0xB8, -2: 0xC0, -3: 0xC4, -4: 0xC8}


def _int_operands(rng, m, n, k):
    xi = rng.integers(-4, 5, size=(m, k))
    wi = rng.integers(-4, 5, size=(n, k))
    xq = np.vectorize(INT_CODES.get)(xi).astype(np.uint8)
    wq = np.vectorize(INT_CODES.get)(wi).astype(np.uint8)
    return xi, wi, xq, wq


def test_integer_operands_exact():
    # small integers are exact E4M3 values: with unit scales the projection is
    # an integer matrix product, compared exactly with Python integers
    rng = np.random.default_rng(0)
    xi, wi, xq, wq = _int_operands(rng, 7, 5, 96)
    y = oracle.w8a8_gemm(xq, np.ones(7, np.float32), wq, np.ones(5, np.float32))
    ref = [[sum(int(a) * int(b) for a, b in zip(xi[m], wi[n])) for n in range(5)] for m in range(7)]
    assert np.array_equal(y, np.array(ref, dtype=np.float64))


def test_brute_force_with_scales():
    # triple loop over decoded codes and the scale definition, tiny shape
    rng = np.random.default_rng(1)
    xq = rng.integers(0, 256, size=(3, 6)).astype(np.uint8)
    wq = rng.integers(0, 256, size=(4, 6)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x10  # no NaN codes
    wq[(wq & 0x7F) == 0x7F] = 0x21
    sx = rng.uniform(0.1, 2.0, 3).astype(np.float32)
    sw = rng.uniform(0.1, 2.0, 4).astype(np.float32)
    dx = oracle.e4m3_decode(xq)
    dw = oracle.e4m3_decode(wq)
    y = oracle.w8a8_gemm(xq, sx, wq, sw)
    for m in range(3):
        for n in range(4):
            acc = 0.0
            for k in range(6):
                acc += float(dx[m, k]) * float(dw[n, k])
            assert y[m, n] == pytest.approx(acc * float(sx[m]) * float(sw[n]), rel=1e-14, abs=1e-300)


def test_scales_factor_exactly():
    rng = np.random.default_rng(2)
    _, _, xq, wq = _int_operands(rng, 6, 5, 64)
    sx = rng.uniform(0.5, 1.5, 6).astype(np.float32)
    sw = rng.uniform(0.5, 1.5, 5).astype(np.float32)
    y = oracle.w8a8_gemm(xq, sx, wq, sw)
    sx2 = sx.copy(); sx2[2] *= 2
    sw2 = sw.copy(); sw2[4] *= 4
    y2 = oracle.w8a8_gemm(xq, sx2, wq, sw2)
    expect = y.copy(); expect[2, :] *= 2; expect[:, 4] *= 4
    assert np.array_equal(y2, expect)


def test_quantised_projection_close_to_float_projection():
    # per-row quantisation of both operands: each dequantised value is within
    # 2^-4 relative (normal range) or 2^-10 * scale of the original, so the
    # projection error is bounded by sum_k of those per-term errors
    rng = np.random.default_rng(3)
    m, n, k = 16, 12, 256
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = (rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # truncation: still bf16 values
    xb, wb = to_bits(x), to_bits(w)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xq, sx = oracle.quant_fp8_per_token(xb)
    wq, sw = oracle.quant_weight_per_channel(wb)
    y = oracle.w8a8_gemm(xq, sx, wq, sw)
    exact = xf @ wf.T
    ex = np.abs(oracle.e4m3_decode(xq) * sx[:, None].astype(np.float64) - xf)
    ew = np.abs(oracle.e4m3_decode(wq) * sw[:, None].astype(np.float64) - wf)
    bound = ex @ np.abs(wf).T + np.abs(xf) @ ew.T + ex @ ew.T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-9) + 1e-12)
    assert np.all(ex <= np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sx[:, None]) * (1 + 1e-6))
