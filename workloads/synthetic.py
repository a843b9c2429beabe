"""Seeded synthetic inputs shaped like the Wan video-DiT attention layers.

This module only draws numbers. It holds none of the attention or
quantisation arithmetic: both the CPU oracle and the HIP path receive the
arrays it returns and nothing else from it.

Shapes follow the workloads on the pages: Wan2.1 latent grids of
21 x 30 x 52 (480P) and 21 x 45 x 80 (720P, 81 frames) tokens, 12 heads
(1.3B) or 40 heads (14B) of width 128, and 5120-wide activations.

Recipe (numpy PCG64 streams, fixed draw order):
  1. from the stream seeded by `seed`: four frequency triples f^m drawn
     without replacement from {0,1,2}^3 minus the zero triple, shared by
     Q, K and V; then per tensor X in (Q, K, V) the phases
     phi[m, head, chan] ~ U[0, 2 pi);
  2. noise z ~ N(0, 1), drawn per (tensor, batch, run of 4096 tokens) from
     the stream seeded by SeedSequence(seed, spawn_key=(tensor, batch, run))
     so that runs can be drawn in parallel;
     X = 0.5 z + sum_m 0.5 sin(2 pi (f_t t/T + f_h h/Hg + f_w w/Wg) + phi),
     with token i at raster position (t, h, w), i = (t*Hg + h)*Wg + w;
  3. values rounded to bfloat16 (round to nearest even).
Low-rank projection matrices are N(0, 1/d) (separate stream). The per-token
gate is drawn directly from the distribution that a near-zero-initialised
gate projection gives: g = 0.05 + 0.1 z ("amplified" runs: g = 1 + z).
Activations for the FP8 quantiser are Student-t (nu = 4) with 1% of the
channels scaled by 20 (outlier channels).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    d: int
    T: int
    Hg: int
    Wg: int
    block_q: int
    block_k: int
    sparsity: float
    rank: int

    @property
    def L(self) -> int:
        return self.T * self.Hg * self.Wg


# The attention workloads. Block sizes of the two 14B layers are not stated
# on the pages; they take the 128-query x 64-key blocks of the 1.3B layer.
TINY = AttnConfig("tiny-1024", 1, 2, 64, 4, 16, 16, 64, 64, 0.75, 16)
WAN13B_480P = AttnConfig("wan1.3b-480p", 1, 12, 128, 21, 30, 52, 128, 64, 0.90, 32)
WAN14B_480P = AttnConfig("wan14b-480p", 1, 40, 128, 21, 30, 52, 128, 64, 0.95, 32)
WAN14B_720P = AttnConfig("wan14b-720p", 1, 40, 128, 21, 45, 80, 128, 64, 0.97, 32)
WAN14B_720P_S90 = dataclasses.replace(WAN14B_720P, name="wan14b-720p-s0.90", sparsity=0.90)

CONFIGS = {c.name: c for c in (TINY, WAN13B_480P, WAN14B_480P, WAN14B_720P, WAN14B_720P_S90)}

# Activation shapes for the per-token FP8 quantiser: one 480P and one 720P
# token count, 5120 channels (the 14B model width).
QUANT_480P = (32760, 5120)
QUANT_720P = (75600, 5120)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in chunks to bound temporaries on very large tensors
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step].astype(np.uint64)
        nan = (v & 0x7FFFFFFF) > 0x7F800000
        r = (v + 0x7FFF + ((v >> 16) & 1)) >> 16
        r = np.where(nan, (v >> 16) | 0x40, r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def _positions(cfg: AttnConfig):
    i = np.arange(cfg.L)
    t = i // (cfg.Hg * cfg.Wg)
    h = (i // cfg.Wg) % cfg.Hg
    w = i % cfg.Wg
    return t, h, w


_CHUNK = 4096


def _pool():
    import concurrent.futures as cf
    import os
    return cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))


def _child(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def gen_qkv(cfg: AttnConfig, seed: int = 0):
    """Q, K, V as bfloat16 bit patterns (uint16), layout [B, L, H, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    triples = [(a, b, c) for a in range(3) for b in range(3) for c in range(3) if (a, b, c) != (0, 0, 0)]
    pick = rng.choice(len(triples), size=4, replace=False)
    freqs = np.array([triples[p] for p in pick], dtype=np.float64)  # [4, 3]
    t, h, w = _positions(cfg)
    ang = 2.0 * math.pi * (np.outer(t / cfg.T, freqs[:, 0]) + np.outer(h / cfg.Hg, freqs[:, 1])
                           + np.outer(w / cfg.Wg, freqs[:, 2]))  # [L, 4]
    basis = np.concatenate([np.sin(ang), np.cos(ang)], axis=1).astype(np.float32)  # [L, 8]
    HD = cfg.H * cfg.d
    coefs = []
    for _ in range(3):
        phase = rng.uniform(0.0, 2.0 * math.pi, size=(4, HD))
        # sin(a + p) = sin a cos p + cos a sin p
        coefs.append(0.5 * np.concatenate([np.cos(phase), np.sin(phase)], axis=0).astype(np.float32))  # [8, HD]
    out = [np.empty((cfg.B, cfg.L, HD), dtype=np.uint16) for _ in range(3)]

    def work(job):
        x_i, b, s0 = job
        e0 = min(cfg.L, s0 + _CHUNK)
        x = basis[s0:e0] @ coefs[x_i]
        x += 0.5 * _child(seed, x_i, b, s0 // _CHUNK).standard_normal(size=(e0 - s0, HD), dtype=np.float32)
        out[x_i][b, s0:e0] = f32_to_bf16_bits(x)

    jobs = [(x_i, b, s0) for x_i in range(3) for b in range(cfg.B) for s0 in range(0, cfg.L, _CHUNK)]
    with _pool() as ex:
        list(ex.map(work, jobs))
    return tuple(o.reshape(cfg.B, cfg.L, cfg.H, cfg.d) for o in out)


def gen_lowrank_params(cfg: AttnConfig, seed: int = 0):
    """P_q, P_k (bf16 bits, [rank, d]) drawn N(0, 1/d), shared by all heads."""
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    std = 1.0 / math.sqrt(cfg.d)
    pq = rng.standard_normal(size=(cfg.rank, cfg.d)) * std
    pk = rng.standard_normal(size=(cfg.rank, cfg.d)) * std
    return f32_to_bf16_bits(pq.astype(np.float32)), f32_to_bf16_bits(pk.astype(np.float32))


def gen_gate(cfg: AttnConfig, seed: int = 0, amplified: bool = False) -> np.ndarray:
    """Per-token gate, float32 [B, L] (one scalar per token, shared by heads)."""
    rng = np.random.Generator(np.random.PCG64(seed + 2_000_003))
    z = rng.standard_normal(size=(cfg.B, cfg.L))
    g = (1.0 + z) if amplified else (0.05 + 0.1 * z)
    return g.astype(np.float32)


def gen_activation(M: int, K: int, seed: int = 0, outlier_frac: float = 0.01,
                   outlier_gain: float = 20.0) -> np.ndarray:
    """bf16 bits [M, K]: Student-t (nu=4) values, a fixed 1% of channels x20.

    The outlier channels come from the stream seeded by seed + 3000003; the
    values of each run of rows from SeedSequence(seed + 3000003,
    spawn_key=(run,)).
    """
    base = seed + 3_000_003
    rng = np.random.Generator(np.random.PCG64(base))
    n_out = max(1, int(round(outlier_frac * K)))
    chans = rng.choice(K, size=n_out, replace=False)
    gain = np.ones(K, dtype=np.float32)
    gain[chans] = outlier_gain
    out = np.empty((M, K), dtype=np.uint16)
    step = max(1, (1 << 22) // K)

    def work(s0):
        e0 = min(M, s0 + step)
        x = _child(base, s0 // step).standard_t(4.0, size=(e0 - s0, K)).astype(np.float32) * gain
        out[s0:e0] = f32_to_bf16_bits(x)

    with _pool() as ex:
        list(ex.map(work, range(0, M, step)))
    return out


# Config-5 projections of the 720P block: QKV (3 x 5120 outputs) and output.
PROJ_QKV_720P = (75600, 15360, 5120)  # (M tokens, N outputs, K inputs)
PROJ_OUT_720P = (75600, 5120, 5120)


def gen_weight(N: int, K: int, seed: int = 0) -> np.ndarray:
    """bf16 bits [N, K] ~ N(0, 1/K) (one row per output channel), from the
    stream seeded by seed + 4000003 (rows in runs, like gen_activation)."""
    base = seed + 4_000_003
    out = np.empty((N, K), dtype=np.uint16)
    step = max(1, (1 << 22) // K)

    def work(s0):
        e0 = min(N, s0 + step)
        w = (_child(base, s0 // step).standard_normal((e0 - s0, K)) / np.sqrt(K)).astype(np.float32)
        out[s0:e0] = f32_to_bf16_bits(w)

    with _pool() as ex:
        list(ex.map(work, range(0, N, step)))
    return out


def gen_fp8_codes(M: int, K: int, seed: int = 0):
    """(uint8 [M, K] random finite E4M3FN codes, float32 [M] scales in
    [2^-8, 2^-4)): operands of the projection at full size, drawn directly
    (stream seed + 5000003)."""
    base = seed + 5_000_003
    out = np.empty((M, K), dtype=np.uint8)
    step = max(1, (1 << 23) // K)

    def work(s0):
        e0 = min(M, s0 + step)
        c = _child(base, s0 // step).integers(0, 254, size=(e0 - s0, K), dtype=np.uint8)
        c[c >= 0x7F] += 1  # skip 0x7F (NaN); 254 values map onto 0..0xFE minus 0x7F
        out[s0:e0] = c
    with _pool() as ex:
        list(ex.map(work, range(0, M, step)))
    rng = np.random.Generator(np.random.PCG64(base))
    scales = np.exp2(rng.uniform(-8.0, -4.0, M)).astype(np.float32)
    return out, scales


def gen_qk_rows(M: int, C: int, seed: int = 0) -> np.ndarray:
    """bf16 bits [M, C]: rows of a q or k projection, N(0, 1) times a per-row
    scale 2^U(-3, 3) (stream seed + 6000007, rows in runs)."""
    base = seed + 6_000_007
    out = np.empty((M, C), dtype=np.uint16)
    step = max(1, (1 << 22) // C)

    def work(s0):
        e0 = min(M, s0 + step)
        rng = _child(base, s0 // step)
        scale = np.exp2(rng.uniform(-3.0, 3.0, size=(e0 - s0, 1)))
        out[s0:e0] = f32_to_bf16_bits((rng.standard_normal((e0 - s0, C)) * scale).astype(np.float32))

    with _pool() as ex:
        list(ex.map(work, range(0, M, step)))
    return out


def gen_norm_weight(C: int, seed: int = 0) -> np.ndarray:
    """bf16 bits [C]: an RMSNorm weight 1 + 0.1 N(0, 1) (stream seed + 7000003)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7_000_003))
    return f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32))


def gen_gate_weight(K: int, seed: int = 0) -> np.ndarray:
    """bf16 bits [K]: the gate projection weight, N(0, 1e-2 / K) (variance
    notation, stream seed + 8000009); the bias is 0.05."""
    rng = np.random.Generator(np.random.PCG64(seed + 8_000_009))
    return f32_to_bf16_bits((rng.standard_normal(K) * np.sqrt(1e-2 / K)).astype(np.float32))


GATE_BIAS = 0.05
