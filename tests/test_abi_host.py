"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point declared in include/sd.h, its host helpers agree with the
oracle's readings, and argument validation rejects bad calls before any
device work (no pointer below is ever dereferenced).
"""
import ctypes
import os
import re

import pytest

import oracle
import sparse_rank_attention_rola_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "sd.h")).read()
    return sorted(set(re.findall(r"\b(sd_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sd.lib()
    declared = _declared_symbols()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(sd.EXPORTED) == declared


def test_keep_count_matches_oracle():
    for s in (0.0, 0.5, 0.75, 0.9, 0.95, 0.97, 0.99):
        for n in (1, 16, 100, 512, 1182, 2048):
            assert sd.sd_keep_count(s, n) == oracle.keep_count(s, n), (s, n)
    assert sd.sd_keep_count(1.0, 10) == -1
    assert sd.sd_keep_count(0.5, 0) == -1


@pytest.mark.parametrize("rank", [16, 32])
def test_rope_default_matches_oracle_reading(rank):
    mine = sd.sd_rope_default(rank)
    ref = oracle.rope_pairs(rank)
    assert [(d, a) for d, a, _ in mine] == [(d, a) for d, a, _ in ref]
    for (_, _, t1), (_, _, t2) in zip(mine, ref):
        assert abs(t1 - t2) <= 2 ** -23 * t2


def test_status_strings():
    lib = sd.lib()
    for code in range(6):
        assert lib.sd_status_string(code)
    assert lib.sd_status_string(99) == b"unknown status"


# --- validation: every call below must fail on the host -------------------

FAKE = 1 << 20  # 16-byte aligned, never dereferenced


def _shape(**kw):
    B, H, L, d = kw.get("B", 1), kw.get("H", 2), kw.get("L", 1024), kw.get("d", 64)
    grid = kw.get("grid", (4, 16, 16))
    s = sd.sd_attn_shape(B, H, L, d, grid[0], grid[1], grid[2], kw.get("bq", 64), kw.get("bk", 64))
    st = (L * H * d, H * d, d)
    for pre in ("sq", "sk", "sv", "so"):
        setattr(s, pre + "_b", st[0])
        setattr(s, pre + "_l", kw.get("sl", st[1]))
        setattr(s, pre + "_h", st[2])
    return s


def _lr(rank=16, pairs=None, eps=1e-6, phi=1, rms_weight=None):
    pairs = pairs if pairs is not None else sd.sd_rope_default(rank)
    arr = (sd.sd_rope_pair * max(1, len(pairs)))(*[sd.sd_rope_pair(d, a, t) for d, a, t in pairs])
    p = sd.sd_lowrank_params(rank, phi, FAKE, FAKE, 0, ctypes.cast(arr, ctypes.POINTER(sd.sd_rope_pair)),
                             len(pairs), eps, rms_weight)
    return p, arr


host_only = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="host-only validation tests run where no GPU is visible")


def _call_select(s, k=4, ws_bytes=1 << 30, Q=FAKE, idx=FAKE, ws=FAKE):
    return sd.lib().sd_block_select(ctypes.byref(s), Q, FAKE, k, idx, ws, ws_bytes, None)


@host_only
def test_block_select_validation():
    lib = sd.lib()
    assert _call_select(_shape(d=96)) == sd.SD_ERR_UNSUPPORTED
    assert _call_select(_shape(bq=32)) == sd.SD_ERR_UNSUPPORTED
    assert _call_select(_shape(bk=128)) == sd.SD_ERR_UNSUPPORTED
    assert _call_select(_shape(L=0)) == sd.SD_ERR_INVALID_ARG
    assert _call_select(_shape(L=200000, grid=(1, 1, 200000))) == sd.SD_ERR_UNSUPPORTED
    assert _call_select(_shape(sl=100)) == sd.SD_ERR_ALIGN
    assert _call_select(_shape(), Q=None) == sd.SD_ERR_INVALID_ARG
    assert _call_select(_shape(), Q=FAKE + 2) == sd.SD_ERR_ALIGN
    assert _call_select(_shape(), k=0) == sd.SD_ERR_INVALID_ARG
    assert _call_select(_shape(), k=17) == sd.SD_ERR_INVALID_ARG
    need = lib.sd_block_select_workspace_size(ctypes.byref(_shape()))
    assert need > 0
    assert _call_select(_shape(), ws_bytes=need - 1) == sd.SD_ERR_WORKSPACE
    assert _call_select(_shape(), ws=None) == sd.SD_ERR_WORKSPACE
    assert _call_select(_shape(), ws=FAKE + 16) == sd.SD_ERR_ALIGN
    assert b"workspace" in lib.sd_last_error() or b"aligned" in lib.sd_last_error()
    assert lib.sd_block_select(None, FAKE, FAKE, 4, FAKE, FAKE, 1 << 30, None) == sd.SD_ERR_INVALID_ARG


@host_only
def test_sparse_attn_validation():
    lib = sd.lib()
    s = _shape()
    call = lambda **kw: lib.sd_sparse_attn(ctypes.byref(kw.get("s", s)), FAKE, FAKE, kw.get("V", FAKE), FAKE,
                                           kw.get("k", 4), kw.get("scale", 0.125), FAKE, kw.get("dt", 2),
                                           kw.get("rms", None), None)
    assert call(V=None) == sd.SD_ERR_INVALID_ARG
    assert call(k=0) == sd.SD_ERR_INVALID_ARG
    assert call(k=100) == sd.SD_ERR_INVALID_ARG
    assert call(scale=0.0) == sd.SD_ERR_INVALID_ARG
    assert call(scale=float("nan")) == sd.SD_ERR_INVALID_ARG
    assert call(dt=7) == sd.SD_ERR_INVALID_ARG
    assert call(rms=FAKE + 1) == sd.SD_ERR_ALIGN
    assert call(s=_shape(d=32)) == sd.SD_ERR_UNSUPPORTED


@host_only
def test_lowrank_validation():
    lib = sd.lib()
    s = _shape()

    def call(shape=s, lr=None, ws_bytes=1 << 30, dt=2):
        p, keep = lr if lr is not None else _lr()
        return lib.sd_lowrank_attn(ctypes.byref(shape), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, dt, None, FAKE,
                                   ws_bytes, None)

    assert call(shape=_shape(grid=(4, 16, 15))) == sd.SD_ERR_INVALID_ARG  # T*Hg*Wg != L
    assert call(lr=_lr(rank=24)) == sd.SD_ERR_UNSUPPORTED
    assert call(lr=_lr(phi=2)) == sd.SD_ERR_UNSUPPORTED
    assert call(lr=_lr(pairs=[(15, 0, 1.0)])) == sd.SD_ERR_INVALID_ARG  # dim+1 out of range
    assert call(lr=_lr(pairs=[(0, 3, 1.0)])) == sd.SD_ERR_INVALID_ARG  # bad axis
    assert call(lr=_lr(pairs=[(0, 0, 1.0), (1, 1, 1.0)])) == sd.SD_ERR_INVALID_ARG  # overlap
    assert call(lr=_lr(eps=-1.0)) == sd.SD_ERR_INVALID_ARG
    assert call(lr=_lr(rms_weight=FAKE + 2)) == sd.SD_ERR_ALIGN  # the weight is read 4 channels at a time
    assert call(dt=0) == sd.SD_ERR_INVALID_ARG
    need = lib.sd_lowrank_workspace_size(ctypes.byref(s), ctypes.byref(_lr()[0]))
    assert need > 0
    assert call(ws_bytes=need - 1) == sd.SD_ERR_WORKSPACE


@host_only
def test_gate_fuse_and_quant_validation():
    lib = sd.lib()
    s = _shape()
    assert lib.sd_gate_fuse(ctypes.byref(s), FAKE, FAKE, 2, None, 0, 1, 0, FAKE, None) == sd.SD_ERR_INVALID_ARG
    assert lib.sd_gate_fuse(ctypes.byref(s), FAKE, FAKE, 2, FAKE, -1, 1, 0, FAKE, None) == sd.SD_ERR_INVALID_ARG
    assert lib.sd_gate_fuse(ctypes.byref(s), FAKE, FAKE, 9, FAKE, 0, 1, 0, FAKE, None) == sd.SD_ERR_INVALID_ARG
    q = lambda M, K, ldx, ldq, x=FAKE, qq=FAKE: lib.sd_quant_fp8_per_token(x, M, K, ldx, qq, ldq, FAKE, None)
    assert q(10, 100, 104, 104) == sd.SD_ERR_ALIGN  # K % 8
    assert q(10, 128, 132, 128) == sd.SD_ERR_ALIGN  # ldx % 8
    assert q(10, 32768, 32768, 32768) == sd.SD_ERR_UNSUPPORTED
    assert q(10, 128, 64, 128) == sd.SD_ERR_INVALID_ARG  # ldx < K
    assert q(-1, 128, 128, 128) == sd.SD_ERR_INVALID_ARG
    assert q(10, 128, 128, 128, x=None) == sd.SD_ERR_INVALID_ARG
    assert q(10, 128, 128, 128, qq=FAKE + 4) == sd.SD_ERR_ALIGN
    # no rows: nothing to do, NULL pointers accepted, nothing launched
    assert lib.sd_quant_fp8_per_token(None, 0, 128, 128, None, 128, None, None) == sd.SD_OK
    assert lib.sd_quant_fp8_gate(None, 0, 128, 128, None, 128, None, None, 0.0, None, None) == sd.SD_OK
    assert q(0, 100, 104, 104) == sd.SD_ERR_ALIGN  # the shape rules still apply


@host_only
def test_quant_gate_validation():
    lib = sd.lib()

    def c(M=10, K=128, ldx=128, ldq=128, x=FAKE, w=FAKE, g=FAKE, b=0.05):
        return lib.sd_quant_fp8_gate(x, M, K, ldx, FAKE, ldq, FAKE, w, b, g, None)

    assert c(K=4) == sd.SD_ERR_INVALID_ARG
    assert c(K=132, ldx=136, ldq=136) == sd.SD_ERR_ALIGN
    assert c(K=32768, ldx=32768, ldq=32768) == sd.SD_ERR_UNSUPPORTED
    assert c(ldx=64) == sd.SD_ERR_INVALID_ARG
    assert c(b=float("nan")) == sd.SD_ERR_INVALID_ARG
    assert c(w=None) == sd.SD_ERR_INVALID_ARG
    assert c(w=FAKE + 2) == sd.SD_ERR_ALIGN
    assert c(g=FAKE + 2) == sd.SD_ERR_ALIGN


@host_only
def test_gemm_fp8_validation():
    lib = sd.lib()

    def g(M=300, N=200, K=128, ldx=128, ldw=128, ldy=200, xq=FAKE, y=FAKE):
        return lib.sd_gemm_fp8_w8a8(xq, M, K, ldx, FAKE, FAKE, N, ldw, FAKE, y, ldy, None)

    assert g(K=100, ldx=112, ldw=112) == sd.SD_ERR_UNSUPPORTED  # K % 64
    assert g(K=131072, ldx=131072, ldw=131072) == sd.SD_ERR_UNSUPPORTED
    assert g(ldx=64) == sd.SD_ERR_INVALID_ARG  # ldx < K
    assert g(ldy=100) == sd.SD_ERR_INVALID_ARG  # ldy < N
    assert g(ldx=136) == sd.SD_ERR_ALIGN  # ldx % 16
    assert g(ldy=202) == sd.SD_ERR_ALIGN  # ldy % 4
    assert g(M=-1) == sd.SD_ERR_INVALID_ARG
    assert g(xq=None) == sd.SD_ERR_INVALID_ARG
    assert g(xq=FAKE + 8) == sd.SD_ERR_ALIGN
    assert g(y=FAKE + 4) == sd.SD_ERR_ALIGN
    assert g(ldx=1 << 24, ldw=1 << 24) == sd.SD_ERR_UNSUPPORTED
    assert g(M=0) == sd.SD_OK  # nothing to do, nothing touched


@host_only
def test_qk_norm_rope_validation():
    lib = sd.lib()
    pairs = sd.sd_rope_default(128)
    rp = (sd.sd_rope_pair * 64)(*[sd.sd_rope_pair(a, b, c) for a, b, c in pairs])
    rptr = ctypes.cast(rp, ctypes.POINTER(sd.sd_rope_pair))
    odd = (sd.sd_rope_pair * 1)(sd.sd_rope_pair(43, 2, 1.0))

    def c(B=1, L=60, H=4, d=128, T=3, Hg=4, Wg=5, q=FAKE, ld=512, eps=1e-6, rope=rptr, n=64, gq=None, Q=FAKE,
          qm=None, bq=128, bk=64):
        return lib.sd_qk_norm_rope(B, L, H, d, T, Hg, Wg, q, FAKE, ld, gq, None, eps, rope, n, Q, FAKE, FAKE, FAKE,
                                   qm, None, bq, bk, None)

    assert c(qm=FAKE, bq=32) == sd.SD_ERR_UNSUPPORTED  # block means: block_q in {64, 128}
    assert c(qm=FAKE, bk=128) == sd.SD_ERR_UNSUPPORTED  # block_k = 64
    assert c(qm=FAKE + 4) == sd.SD_ERR_ALIGN

    assert c(d=96) == sd.SD_ERR_UNSUPPORTED
    assert c(H=80) == sd.SD_ERR_UNSUPPORTED  # H*d > 8192
    assert c(L=61) == sd.SD_ERR_INVALID_ARG  # T*Hg*Wg != L
    assert c(ld=256) == sd.SD_ERR_INVALID_ARG  # ld_in < H*d
    assert c(ld=516) == sd.SD_ERR_ALIGN
    assert c(eps=-1.0) == sd.SD_ERR_INVALID_ARG
    assert c(n=65) == sd.SD_ERR_INVALID_ARG
    assert c(d=64, H=8, rope=ctypes.cast(odd, ctypes.POINTER(sd.sd_rope_pair)), n=1) == sd.SD_ERR_INVALID_ARG
    assert c(q=None) == sd.SD_ERR_INVALID_ARG
    assert c(Q=FAKE + 8) == sd.SD_ERR_ALIGN
    assert c(gq=FAKE + 2) == sd.SD_ERR_ALIGN


@host_only
def test_rola_validation():
    lib = sd.lib()
    s = _shape()
    p, keep = _lr()
    need = lib.sd_rola_workspace_size(ctypes.byref(s), ctypes.byref(p), 4)
    assert need >= lib.sd_block_select_workspace_size(ctypes.byref(s))

    def call(k=4, ws_bytes=need, g=FAKE, Qn=None, shape=s):
        return lib.sd_rola_attention(ctypes.byref(shape), ctypes.byref(p), FAKE, FAKE, FAKE, Qn, None, g, 0, 1, 0, k,
                                     0.125, FAKE, None, FAKE, ws_bytes, None)

    assert call(k=0) == sd.SD_ERR_INVALID_ARG
    assert call(g=None) == sd.SD_ERR_INVALID_ARG
    assert call(Qn=FAKE + 8) == sd.SD_ERR_ALIGN
    assert call(ws_bytes=need - 1) == sd.SD_ERR_WORKSPACE
    assert call(shape=_shape(grid=(1, 1, 1))) == sd.SD_ERR_INVALID_ARG
    assert lib.sd_rola_workspace_size(ctypes.byref(s), ctypes.byref(p), 0) == 0


@host_only
def test_rola_noalloc_validation():
    # argument errors as for the workspace entry; a shape whose workspace
    # exceeds the static scratch is refused before any device call
    lib = sd.lib()
    p, keep = _lr()

    def call(shape, k=4, g=FAKE):
        return lib.sd_rola_attention_noalloc(ctypes.byref(shape), ctypes.byref(p), FAKE, FAKE, FAKE, None, None, g,
                                             0, 1, 0, k, 0.125, FAKE, None, None)

    assert call(_shape(), k=0) == sd.SD_ERR_INVALID_ARG
    assert call(_shape(), g=None) == sd.SD_ERR_INVALID_ARG
    assert call(_shape(grid=(1, 1, 1))) == sd.SD_ERR_INVALID_ARG
    big = _shape(B=2, H=40, L=75600, d=128, grid=(21, 45, 80), bq=128)
    assert lib.sd_rola_workspace_size(ctypes.byref(big), ctypes.byref(p), 36) > sd.SD_NOALLOC_SCRATCH_BYTES
    assert call(big, k=36) == sd.SD_ERR_UNSUPPORTED
    assert "static buffer" in lib.sd_last_error().decode()


@host_only
def test_variant_fields_validation():
    lib = sd.lib()

    def shp(select=0, chunk=0, window=0, **kw):
        s = _shape(**kw)
        s.select, s.chunk_tokens, s.window = select, chunk, window
        return s

    assert _call_select(shp(select=2)) == sd.SD_ERR_INVALID_ARG
    assert _call_select(shp(chunk=-1)) == sd.SD_ERR_INVALID_ARG
    assert _call_select(shp(chunk=256, window=-1)) == sd.SD_ERR_INVALID_ARG
    assert _call_select(shp(window=2)) == sd.SD_ERR_INVALID_ARG  # a window needs chunks
    assert _call_select(shp(select=1, grid=(1, 1, 1))) == sd.SD_ERR_INVALID_ARG  # the fixed pattern needs the grid
    assert _call_select(shp(chunk=1, L=8192, grid=(8, 32, 32))) == sd.SD_ERR_UNSUPPORTED  # > 4096 chunks
    # a causal window sizes one low-rank state per chunk
    p, keep = _lr()
    one = lib.sd_rola_workspace_size(ctypes.byref(shp()), ctypes.byref(p), 4)
    many = lib.sd_rola_workspace_size(ctypes.byref(shp(chunk=256, window=2)), ctypes.byref(p), 4)
    assert many > one > 0
    # chunks longer than the sequence are the bidirectional layer
    assert lib.sd_rola_workspace_size(ctypes.byref(shp(chunk=5000)), ctypes.byref(p), 4) == one


@host_only
def test_backward_validation():
    lib = sd.lib()
    s = _shape()
    p, keep = _lr()
    need = lib.sd_rola_backward_workspace_size(ctypes.byref(s), ctypes.byref(p), 4)
    assert need > lib.sd_rola_workspace_size(ctypes.byref(s), ctypes.byref(p), 4)

    def call(k=4, ws_bytes=need, Qn=None, dQn=None, idx=FAKE, dO=FAKE, dV=FAKE, g=FAKE, dg=None, saved=None,
             gs=(0, 1, 0)):
        return lib.sd_rola_backward(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, Qn, None, g, *gs, k,
                                    0.125, idx, saved, dO, FAKE, FAKE, dV, dQn, None, None, None, dg, FAKE, ws_bytes,
                                    None)

    assert call(k=0) == sd.SD_ERR_INVALID_ARG
    assert call(idx=None) == sd.SD_ERR_INVALID_ARG
    assert call(dO=None) == sd.SD_ERR_INVALID_ARG
    assert call(dV=None) == sd.SD_ERR_INVALID_ARG
    assert call(g=None) == sd.SD_ERR_INVALID_ARG
    assert call(Qn=FAKE) == sd.SD_ERR_INVALID_ARG  # dQn must come with Qn
    assert call(dQn=FAKE) == sd.SD_ERR_INVALID_ARG
    assert call(Qn=FAKE, dQn=FAKE + 4) == sd.SD_ERR_ALIGN
    assert call(dg=FAKE + 2) == sd.SD_ERR_ALIGN
    # gate strides whose tokens and heads overlap: dg elements would race
    assert s.H > 1 and s.L > 1
    assert call(dg=FAKE, gs=(0, 1, 1)) == sd.SD_ERR_UNSUPPORTED
    assert call(dg=FAKE, gs=(0, 2, 3)) == sd.SD_ERR_UNSUPPORTED
    # without dg the same gate is only read; broadcasts are fine with dg
    assert lib.sd_rola_backward_workspace_size(ctypes.byref(s), ctypes.byref(p), 4) == need
    assert call(ws_bytes=need - 1) == sd.SD_ERR_WORKSPACE
    assert call(saved=ctypes.byref(sd.sd_rola_saved(FAKE, None, FAKE))) == sd.SD_ERR_INVALID_ARG
    assert call(saved=ctypes.byref(sd.sd_rola_saved(FAKE + 2, FAKE, FAKE))) == sd.SD_ERR_ALIGN
    assert lib.sd_rola_backward_workspace_size(ctypes.byref(s), ctypes.byref(p), 0) == 0
    # the saving forward checks its struct too
    assert lib.sd_rola_apply_save(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, 0, 1, 0, 4, 0.125,
                                  FAKE, None, FAKE, 1 << 30, None, None) == sd.SD_ERR_INVALID_ARG
