"""Helpers of the GPU parity tests: device upload of bf16 bit patterns and
the acceptance checks (block map bit-exact outside the tie window, float
outputs within max-abs 2e-2 and relative L2 1e-2)."""
import sys

import numpy as np
import torch

import oracle

MAX_ABS = 2e-2
REL_L2 = 1e-2
TIE_REL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def dev_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, name, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    ma = float(err.max()) if err.size else 0.0
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    say(f"  {name}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, f"{name}: max_abs {ma:.3e} rel_l2 {rl:.3e}"


def block_map_diff(idx_gpu: np.ndarray, S: np.ndarray, k: int):
    """Compare one head's GPU block map [Nq, k] with the oracle's scores.

    Returns (mismatches, ties, rows_differing): a block present in one map
    and not the other is a tie when its score is within 1e-6 * max(1, |tau|)
    of tau, the oracle's k-th largest score of that row; otherwise it is a
    mismatch. Rows must be strictly ascending.
    """
    ref = oracle.topk_block_map(S, k)
    mism = ties = rows = 0
    for b in range(S.shape[0]):
        g = idx_gpu[b]
        assert (np.diff(g) > 0).all(), f"row {b} not strictly ascending: {g}"
        assert g.min() >= 0 and g.max() < S.shape[1]
        if np.array_equal(g, ref[b]):
            continue
        rows += 1
        tau = np.sort(S[b])[::-1][k - 1]
        for c in set(g.tolist()) ^ set(ref[b].tolist()):
            if abs(S[b, c] - tau) <= TIE_REL * max(1.0, abs(tau)):
                ties += 1
            else:
                mism += 1
    return mism, ties, rows


def fp8_code_steps(got: np.ndarray, ref: np.ndarray, name: str, max_step: int = 1) -> int:
    """E4M3 codes against the oracle's: the sign-magnitude code index may
    differ by at most `max_step` (-0 equals +0). Prints and returns the
    number of codes that differ."""
    def index(c):
        c = np.asarray(c, dtype=np.int64)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    d = np.abs(index(got) - index(ref))
    n = int((d != 0).sum())
    worst = int(d.max()) if d.size else 0
    say(f"  {name}: {n} of {d.size} codes one step from E4M3(x/s) ({100.0 * n / max(d.size, 1):.3f}%), "
        f"largest difference {worst} step(s)")
    assert worst <= max_step, f"{name}: a code differs by {worst} steps"
    return n
