"""Pins of the FP8 E4M3 oracle against things other than itself.

Exhaustive over the 256 codes; checked against the OCP spec's table points,
against PyTorch's float8_e4m3fn conversion (a library routine; it rounds to
nearest-even but does not saturate, so it is only used inside +-448),
against closed-form error bounds, and the per-row quantiser against the
exact rational quotient x / s rounded by exhaustive search.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode(codes):
    return torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_decode_spec_points():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3fn_spec_points.json")))
    for p in spec["points"]:
        assert oracle.e4m3_decode(p["code"]) == p["value"], p
        assert oracle.e4m3_encode(p["value"]) == p["code"], p
    for c in spec["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(c))


def test_decode_all_codes_match_library():
    codes = np.arange(256)
    mine = oracle.e4m3_decode(codes)
    ref = _torch_decode(codes)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_encode_decode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (127, 255)])
    assert (oracle.e4m3_encode(oracle.e4m3_decode(codes)) == codes).all()


def test_encode_midpoints_and_neighbours_match_library():
    vals = np.sort(oracle.e4m3_decode(np.arange(127)))
    mids = (vals[:-1] + vals[1:]) / 2.0
    # offsets that float32 holds exactly (the library converts from float32)
    eps = np.abs(mids) * 2.0 ** -18
    pts = np.concatenate([vals, mids, mids - eps, mids + eps, [2.0 ** -30, 2.0 ** -11, 3 * 2.0 ** -11]])
    pts = np.concatenate([pts, -pts])
    pts = pts[np.abs(pts) <= 448.0]
    mine = oracle.e4m3_encode(pts)
    assert (pts.astype(np.float32).astype(np.float64) == pts).all()
    ref = torch.tensor(pts.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mine == ref).all(), pts[mine != ref][:10]


def test_encode_rne_at_ties_is_even_code():
    # 1 + 1/16 is halfway between 1.0 (code 56, even) and 1.125 (code 57)
    assert oracle.e4m3_encode(1.0 + 1.0 / 16) == 56
    # 1.125 + 1/16 is halfway between 1.125 (57) and 1.25 (58, even)
    assert oracle.e4m3_encode(1.125 + 1.0 / 16) == 58
    # halfway between the largest subnormal and the smallest normal
    assert oracle.e4m3_encode(7.5 * 2.0 ** -9) == 8
    # half the smallest subnormal rounds to (even) zero
    assert oracle.e4m3_encode(2.0 ** -10) == 0


def test_encode_saturates():
    assert oracle.e4m3_encode(449.0) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(np.nan) == 0x7F


def test_roundtrip_error_bound_random():
    rng = np.random.default_rng(5)
    v = rng.uniform(-448, 448, size=20000) * np.exp2(rng.integers(-14, 1, size=20000))
    back = oracle.e4m3_decode(oracle.e4m3_encode(v))
    normal = np.abs(v) >= 2.0 ** -6
    # relative error of a nearest rounding with 3 mantissa bits is <= 2^-4
    assert (np.abs(back - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal]).all()
    # subnormal spacing is 2^-9, half of it is the bound
    assert (np.abs(back - v)[~normal] <= 2.0 ** -10).all()


def test_quant_rows_closed_form():
    x = synthetic.gen_activation(64, 512, seed=3)
    codes, scales = oracle.quant_fp8_per_token(x)
    xf = oracle.bf16_bits_to_f64(x)
    amax = np.abs(xf).max(axis=1)
    # the scale is amax / 448 to float32 precision
    assert np.allclose(scales, amax / 448.0, rtol=2.0 ** -23, atol=0)
    deq = oracle.e4m3_decode(codes) * scales[:, None].astype(np.float64)
    # each row's largest element lands on +-448 (code 0x7E / 0xFE)
    arg = np.abs(xf).argmax(axis=1)
    assert (codes[np.arange(64), arg] & 0x7F == 0x7E).all()
    # dequantised error: half an E4M3 step, relative to the row scale
    rel = np.abs(deq - xf) / np.maximum(np.abs(xf), 2.0 ** -6 * scales[:, None])
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)


def test_quant_zero_row_and_sign():
    x = np.zeros((2, 16), dtype=np.uint16)
    x[1, 3] = 0xBF80  # -1.0
    codes, scales = oracle.quant_fp8_per_token(x)
    assert (codes[0] == 0).all() and np.isfinite(scales[0]) and scales[0] > 0
    assert codes[1, 3] == 0xFE
    assert scales[1] == np.float32(1.0) / np.float32(448.0)


def _tie_rows(n_cols, seed):
    """Student-t rows plus rows whose |x|max has a bf16 significand that is a
    multiple of 7 (140, 168, 196, 210, 252): 448 / amax then has a factor of
    1/7 and x / s lands exactly on E4M3 rounding midpoints for many x."""
    x = synthetic.gen_activation(12, n_cols, seed)
    xf = oracle.bf16_bits_to_f64(x).astype(np.float32)
    for i, b in enumerate([140, 168, 196, 210, 252, 154, 182]):
        amax = np.float32(b) * np.float32(2.0 ** -5)
        row = np.clip(xf[i], -0.99 * amax, 0.99 * amax)
        row[np.abs(row).argmax()] = -amax if i % 2 else amax
        xf[i] = row
    return synthetic.f32_to_bf16_bits(xf)


def _nearest_code_exact(x, s):
    """E4M3 code of the rational x / s by exhaustive search over the 127
    finite magnitudes, comparing exact fractions: nearest value, ties to the
    even code, anything above 448 saturating to 448."""
    t = Fraction(float(x)) / Fraction(float(s))
    mag = abs(t)
    vals = [Fraction(float(v)) for v in oracle.e4m3_decode(np.arange(127))]
    best = None
    for c, v in enumerate(vals):
        d = abs(mag - v)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    code = best[0]
    if mag >= vals[126]:
        code = 126
    return code | (0x80 if x < 0 or (x == 0 and np.signbit(x)) else 0)


def test_quant_codes_are_exact_nearest_of_quotient():
    # The definition written out independently: the scale from exact amax,
    # then each sampled code from the exact rational x / s.
    x = _tie_rows(384, 11)
    codes, scales = oracle.quant_fp8_per_token(x)
    xf = oracle.bf16_bits_to_f64(x)
    rng = np.random.default_rng(2)
    vals = oracle.e4m3_decode(np.arange(127))
    mids = {Fraction(float(a)) / 2 + Fraction(float(b)) / 2 for a, b in zip(vals[:-1], vals[1:])}
    ties = 0
    for r in range(x.shape[0]):
        amax = max(float(np.abs(xf[r]).max()), float(np.float32(1e-12)))
        assert scales[r] == np.float32(np.float32(amax) / np.float32(448.0))
        cols = rng.choice(x.shape[1], 96, replace=False)
        for c in cols:
            assert codes[r, c] == _nearest_code_exact(xf[r, c], scales[r]), (r, c, xf[r, c])
        ties += sum(1 for c in cols if abs(Fraction(float(xf[r, c])) / Fraction(float(scales[r]))) in mids)
    assert ties > 0, "the sample holds no exact rounding tie"


def test_quant_definition_is_not_the_reciprocal_product():
    # E4M3(x / s) and E4M3(fp32(x * fp32(448 / amax))) differ by one step on
    # some elements of these rows; the oracle must follow the former.
    x = _tie_rows(2048, 12)
    codes, scales = oracle.quant_fp8_per_token(x)
    xf = oracle.bf16_bits_to_f64(x).astype(np.float32)
    amax = np.maximum(np.abs(xf).max(axis=1), np.float32(1e-12)).astype(np.float32)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    recip = oracle.e4m3_encode((xf * inv[:, None]).astype(np.float32).astype(np.float64))
    diff = np.argwhere(recip != codes)
    assert len(diff) > 0
    for r, c in diff[:40]:
        assert codes[r, c] == _nearest_code_exact(float(xf[r, c]), scales[r])
        step = abs(int(codes[r, c] & 0x7F) - int(recip[r, c] & 0x7F))
        assert step == 1 and (codes[r, c] & 0x80) == (recip[r, c] & 0x80)
