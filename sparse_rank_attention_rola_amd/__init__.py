"""Python binding of libsd (RoLA compensated sparse attention + per-token
FP8 quant on MI355X). Argument marshalling only: every step runs in the HIP
kernels of libsd.so; PyTorch provides device memory and the current stream.

The functions carry the names of the C entry points in include/sd.h and
take torch tensors in [B, L, H, d] layout (d contiguous, strides multiples
of 8 elements). If libsd.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SD_LIBRARY", os.path.join(_PKG, "libsd.so"))

SD_OK = 0
SD_ERR_INVALID_ARG = 1
SD_ERR_UNSUPPORTED = 2
SD_ERR_ALIGN = 3
SD_ERR_WORKSPACE = 4
SD_ERR_HIP = 5
SD_NOALLOC_SCRATCH_BYTES = 128 << 20  # the static device scratch of sd_rola_attention_noalloc
SD_DTYPE_BF16 = 1
SD_DTYPE_F32 = 2
SD_PHI_ELU1 = 1
SD_SELECT_TOPK = 0
SD_SELECT_FIXED = 1
_SELECT = {"topk": SD_SELECT_TOPK, "fixed": SD_SELECT_FIXED}

EXPORTED = [
    "sd_keep_count", "sd_rope_default", "sd_block_select_workspace_size", "sd_block_select",
    "sd_sparse_attn", "sd_lowrank_workspace_size", "sd_lowrank_attn", "sd_gate_fuse",
    "sd_quant_fp8_per_token", "sd_quant_fp8_gate", "sd_gemm_fp8_w8a8", "sd_qk_norm_rope", "sd_rola_workspace_size", "sd_rola_attention", "sd_rola_attention_noalloc", "sd_rola_prepare",
    "sd_rola_apply", "sd_rola_apply_save", "sd_rola_backward_workspace_size", "sd_rola_backward",
    "sd_status_string", "sd_last_error",
]


class SdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libsd status {status}: {msg}")
        self.status = status


class sd_attn_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "L", "d", "T", "Hg", "Wg", "block_q", "block_k")] + \
               [(n, ctypes.c_int64) for n in ("sq_b", "sq_l", "sq_h", "sk_b", "sk_l", "sk_h",
                                              "sv_b", "sv_l", "sv_h", "so_b", "so_l", "so_h")] + \
               [(n, ctypes.c_int32) for n in ("select", "chunk_tokens", "window")]


class sd_rola_saved(ctypes.Structure):
    _fields_ = [("Os", ctypes.c_void_p), ("rms", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class sd_rope_pair(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("axis", ctypes.c_int32), ("theta", ctypes.c_float)]


class sd_lowrank_params(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("phi", ctypes.c_int32), ("Pq", ctypes.c_void_p),
                ("Pk", ctypes.c_void_p), ("P_head_stride", ctypes.c_int64),
                ("rope", ctypes.POINTER(sd_rope_pair)), ("n_rope", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rms_weight", ctypes.c_void_p)]


_lib = None
_load_error = None


def _declare(lib):
    P = ctypes.c_void_p
    S = ctypes.POINTER(sd_attn_shape)
    LR = ctypes.POINTER(sd_lowrank_params)
    i32, i64, f32, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "sd_keep_count": (i32, [ctypes.c_double, i32]),
        "sd_rope_default": (i32, [i32, ctypes.c_double, ctypes.POINTER(sd_rope_pair), i32]),
        "sd_block_select_workspace_size": (sz, [S]),
        "sd_block_select": (i32, [S, P, P, i32, P, P, sz, P]),
        "sd_sparse_attn": (i32, [S, P, P, P, P, i32, f32, P, i32, P, P]),
        "sd_lowrank_workspace_size": (sz, [S, LR]),
        "sd_lowrank_attn": (i32, [S, LR, P, P, P, P, i32, P, P, sz, P]),
        "sd_gate_fuse": (i32, [S, P, P, i32, P, i64, i64, i64, P, P]),
        "sd_quant_fp8_per_token": (i32, [P, i64, i64, i64, P, i64, P, P]),
        "sd_quant_fp8_gate": (i32, [P, i64, i64, i64, P, i64, P, P, f32, P, P]),
        "sd_gemm_fp8_w8a8": (i32, [P, i64, i64, i64, P, P, i64, i64, P, P, i64, P]),
        "sd_qk_norm_rope": (i32, [i32, i32, i32, i32, i32, i32, i32, P, P, i64, P, P, f32,
                                  ctypes.POINTER(sd_rope_pair), i32, P, P, P, P, P, P, i32, i32, P]),
        "sd_rola_workspace_size": (sz, [S, LR, i32]),
        "sd_rola_attention": (i32, [S, LR, P, P, P, P, P, P, i64, i64, i64, i32, f32, P, P, P, sz, P]),
        "sd_rola_attention_noalloc": (i32, [S, LR, P, P, P, P, P, P, i64, i64, i64, i32, f32, P, P, P]),
        "sd_rola_prepare": (i32, [S, LR, P, P, P, P, P, P, P, i32, P, P, sz, P]),
        "sd_rola_apply": (i32, [S, LR, P, P, P, P, P, i64, i64, i64, i32, f32, P, P, P, sz, P]),
        "sd_rola_backward_workspace_size": (sz, [S, LR, i32]),
        "sd_rola_apply_save": (i32, [S, LR, P, P, P, P, P, i64, i64, i64, i32, f32, P, P, P, sz, P, P]),
        "sd_rola_backward": (i32, [S, LR, P, P, P, P, P, P, i64, i64, i64, i32, f32, P, P, P, P, P, P, P, P, P, P,
                                   P, P, sz, P]),
        "sd_status_string": (ctypes.c_char_p, [i32]),
        "sd_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded libsd.so; raises if it is not built or does not load."""
    global _lib, _load_error
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def _check(status: int):
    if status != SD_OK:
        raise SdError(status, lib().sd_last_error().decode())


# --------------------------------------------------------------------------
# host helpers
# --------------------------------------------------------------------------

def sd_keep_count(sparsity: float, n_kblocks: int) -> int:
    return lib().sd_keep_count(float(sparsity), int(n_kblocks))


def sd_rope_default(rank: int, base: float = 10000.0):
    buf = (sd_rope_pair * 64)()
    n = lib().sd_rope_default(int(rank), float(base), buf, 64)
    if n < 0:
        raise SdError(SD_ERR_INVALID_ARG, "bad rope arguments")
    return [(buf[i].dim, buf[i].axis, buf[i].theta) for i in range(n)]


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def make_shape(Q, K, V, out_like=None, *, block_q=128, block_k=64, grid=(0, 0, 0), select="topk", chunk_tokens=0,
               window=0) -> sd_attn_shape:
    """sd_attn_shape from [B, L, H, d] tensors (out_like gives the so_* strides).

    select: "topk" (scored) or "fixed" (spatio-temporal pattern); chunk_tokens
    and window: the causal window (0: bidirectional)."""
    B, L, H, d = Q.shape
    T, Hg, Wg = grid
    s = sd_attn_shape(B, H, L, d, T, Hg, Wg, block_q, block_k)
    s.select = _SELECT[select]
    s.chunk_tokens = int(chunk_tokens)
    s.window = int(window)
    o_strides = out_like.stride() if out_like is not None else (L * H * d, H * d, d, 1)
    for pre, st in (("sq", Q.stride()), ("sk", K.stride()), ("sv", V.stride()), ("so", o_strides)):
        if st[3] != 1:
            raise ValueError("the head dimension must be contiguous")
        setattr(s, pre + "_b", st[0])
        setattr(s, pre + "_l", st[1])
        setattr(s, pre + "_h", st[2])
    return s


class LowrankParams:
    """Keeps the ctypes struct and the host RoPE array alive together."""

    def __init__(self, Pq, Pk, rank=None, rope=None, rms_eps=1e-6, rms_weight=None, head_stride=0):
        rank = int(rank if rank is not None else Pq.shape[-2])
        pairs = rope if rope is not None else sd_rope_default(rank)
        self._rope = (sd_rope_pair * max(1, len(pairs)))(*[sd_rope_pair(d, a, t) for d, a, t in pairs])
        self._keep = (Pq, Pk, rms_weight)
        self.p = sd_lowrank_params(rank, SD_PHI_ELU1, Pq.data_ptr(), Pk.data_ptr(), head_stride,
                                   ctypes.cast(self._rope, ctypes.POINTER(sd_rope_pair)), len(pairs),
                                   float(rms_eps), rms_weight.data_ptr() if rms_weight is not None else None)


def _workspace(nbytes: int, device):
    torch = _torch()
    # 256-byte aligned: the caching allocator returns 512-byte aligned blocks
    return torch.empty(max(256, int(nbytes)), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------

def sd_block_select(Q, K, k_keep, *, block_q=128, block_k=64, idx=None, grid=(0, 0, 0), select="topk",
                    chunk_tokens=0, window=0, stream=None):
    """int32 [B, H, Nq, k_keep] block map (ascending rows, -1 padded under a
    causal window); the fixed pattern needs the latent grid."""
    torch = _torch()
    B, L, H, d = Q.shape
    s = make_shape(Q, K, K, block_q=block_q, block_k=block_k, grid=grid, select=select, chunk_tokens=chunk_tokens,
                   window=window)
    nq = -(-L // block_q)
    if idx is None:
        idx = torch.empty((B, H, nq, k_keep), dtype=torch.int32, device=Q.device)
    ws_n = lib().sd_block_select_workspace_size(ctypes.byref(s))
    ws = _workspace(ws_n, Q.device)
    _check(lib().sd_block_select(ctypes.byref(s), _ptr(Q), _ptr(K), int(k_keep), _ptr(idx), _ptr(ws), ws.numel(),
                                 _stream_ptr(stream)))
    return idx


def sd_sparse_attn(Q, K, V, idx, *, block_q=128, block_k=64, sm_scale=None, out_dtype=None, want_rms=True,
                   out=None, chunk_tokens=0, window=0, stream=None):
    """(O_s [B, L, H, d], rms [B, L, H] or None)."""
    torch = _torch()
    B, L, H, d = Q.shape
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, L, H, d), dtype=out_dtype, device=Q.device)
    s = make_shape(Q, K, V, out, block_q=block_q, block_k=block_k, chunk_tokens=chunk_tokens, window=window)
    rms = torch.empty((B, L, H), dtype=torch.float32, device=Q.device) if want_rms else None
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)
    dt = SD_DTYPE_F32 if out.dtype == torch.float32 else SD_DTYPE_BF16
    _check(lib().sd_sparse_attn(ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), int(idx.shape[-1]),
                                float(scale), _ptr(out), dt, _ptr(rms), _stream_ptr(stream)))
    return out, rms


def sd_lowrank_attn(Qn, Kn, V, lr: LowrankParams, *, grid, block_q=128, out_dtype=None, want_C=True, out=None,
                    chunk_tokens=0, window=0, stream=None):
    """(O_lr [B, L, H, d], C or None): C is [B, H, rank, d], or one state
    per autoregressive chunk [B, H, n_chunks, rank, d] under a causal window."""
    torch = _torch()
    B, L, H, d = Qn.shape
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, L, H, d), dtype=out_dtype, device=Qn.device)
    s = make_shape(Qn, Kn, V, out, block_q=block_q, grid=grid, chunk_tokens=chunk_tokens, window=window)
    c_shape = (B, H, lr.p.rank, d) if chunk_tokens <= 0 else (B, H, -(-L // min(chunk_tokens, L)), lr.p.rank, d)
    C = torch.empty(c_shape, dtype=torch.float32, device=Qn.device) if want_C else None
    ws = _workspace(lib().sd_lowrank_workspace_size(ctypes.byref(s), ctypes.byref(lr.p)), Qn.device)
    dt = SD_DTYPE_F32 if out.dtype == torch.float32 else SD_DTYPE_BF16
    _check(lib().sd_lowrank_attn(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Qn), _ptr(Kn), _ptr(V), _ptr(out), dt,
                                 _ptr(C), _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return out, C


def _gate_strides(g, B, L, H):
    if g.dim() == 2:  # [B, L]: one gate per token
        return g.stride(0), g.stride(1), 0
    return g.stride(0), g.stride(1), g.stride(2)


def sd_gate_fuse(Os, Olr, g, *, out=None, stream=None):
    """O = O_s + g * rms(O_s) * O_lr as bf16 [B, L, H, d]; g [B, L] or [B, L, H]."""
    torch = _torch()
    B, L, H, d = Os.shape
    if out is None:
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=Os.device)
    if Olr.stride() != Os.stride() or out.stride() != Os.stride() or Olr.dtype != Os.dtype:
        raise ValueError("Os, Olr and out must share strides and Os/Olr a dtype")
    s = make_shape(Os, Os, Os, Os)
    dt = SD_DTYPE_F32 if Os.dtype == torch.float32 else SD_DTYPE_BF16
    gb, gl, gh = _gate_strides(g, B, L, H)
    _check(lib().sd_gate_fuse(ctypes.byref(s), _ptr(Os), _ptr(Olr), dt, _ptr(g), gb, gl, gh, _ptr(out),
                              _stream_ptr(stream)))
    return out


def sd_quant_fp8_per_token(x, *, q=None, scales=None, stream=None):
    """(codes uint8 [M, K], scales f32 [M]) for bf16 x [M, K]."""
    torch = _torch()
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("rows of x must be contiguous")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().sd_quant_fp8_per_token(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(scales),
                                        _stream_ptr(stream)))
    return q, scales


def sd_quant_fp8_gate(x, w_gate, b_gate, *, q=None, scales=None, g=None, stream=None):
    """Per-token FP8 quant of x (bf16 [M, K]) plus the scalar gate
    g = x @ w_gate + b_gate (w_gate bf16 [K]) in one pass: (q, scales, g)."""
    torch = _torch()
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("rows of x must be contiguous")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    if g is None:
        g = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().sd_quant_fp8_gate(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(scales), _ptr(w_gate),
                                   float(b_gate), _ptr(g), _stream_ptr(stream)))
    return q, scales, g


def sd_gemm_fp8_w8a8(xq, sx, wq, sw, *, out=None, stream=None):
    """bf16 y [M, N] = diag(sx) (E4M3(xq) E4M3(wq)^T) diag(sw) for uint8 codes
    xq [M, K] and wq [N, K] (one row per output channel)."""
    torch = _torch()
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq and wq must have the same K")
    if xq.stride(1) != 1 or wq.stride(1) != 1:
        raise ValueError("rows of xq and wq must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    if out.stride(1) != 1:
        raise ValueError("rows of out must be contiguous")
    _check(lib().sd_gemm_fp8_w8a8(_ptr(xq), M, K, xq.stride(0), _ptr(sx), _ptr(wq), N, wq.stride(0), _ptr(sw),
                                  _ptr(out), out.stride(0), _stream_ptr(stream)))
    return out


def sd_qk_norm_rope(q, k, *, heads, grid, batch=1, gamma_q=None, gamma_k=None, eps=1e-6, rope=None, out=None,
                    block_means=False, block_q=128, block_k=64, means_out=None, stream=None):
    """q/k producer: RMSNorm of every token row of q and k (bf16 [B*L, H*d]
    row views, e.g. slices of the QKV projection's output) and the backbone
    3D RoPE per head. Returns (Q, K, Qn, Kn), bf16 [B, L, H, d] contiguous
    (or the given out tuple); rope defaults to sd_rope_default(d). With
    block_means (or means_out = (qmean, kmean)) it also returns the float64
    block means of Q and K, [B, H, ceil(L / block), d], for sd_rola_prepare."""
    torch = _torch()
    rows, C = q.shape
    if k.shape != q.shape or k.stride() != q.stride():
        raise ValueError("q and k must be row views of the same shape and strides")
    if q.stride(1) != 1:
        raise ValueError("rows of q and k must be contiguous")
    H = int(heads)
    if C % H:
        raise ValueError("H must divide the row length")
    d = C // H
    T, Hg, Wg = grid
    L = rows // batch
    pairs = rope if rope is not None else sd_rope_default(d)
    rp = (sd_rope_pair * max(1, len(pairs)))(*[sd_rope_pair(dm, a, t) for dm, a, t in pairs])
    if out is not None:
        outs = list(out)
        if any(o.shape != (batch, L, H, d) or not o.is_contiguous() or o.dtype != torch.bfloat16 for o in outs):
            raise ValueError("out must be four contiguous bf16 [B, L, H, d] tensors")
    else:
        outs = [torch.empty((batch, L, H, d), dtype=torch.bfloat16, device=q.device) for _ in range(4)]
    means = None
    if means_out is not None:
        means = tuple(means_out)
    elif block_means:
        means = tuple(torch.empty((batch, H, -(-L // bs), d), dtype=torch.float64, device=q.device)
                      for bs in (block_q, block_k))
    _check(lib().sd_qk_norm_rope(batch, L, H, d, T, Hg, Wg, _ptr(q), _ptr(k), q.stride(0),
                                 _ptr(gamma_q) if gamma_q is not None else None,
                                 _ptr(gamma_k) if gamma_k is not None else None, float(eps),
                                 ctypes.cast(rp, ctypes.POINTER(sd_rope_pair)), len(pairs),
                                 *[_ptr(o) for o in outs], _ptr(means[0]) if means else None,
                                 _ptr(means[1]) if means else None, int(block_q), int(block_k),
                                 _stream_ptr(stream)))
    return tuple(outs) + (means if means else ())


def rola_workspace(Q, lr: LowrankParams, k_keep, *, grid, block_q=128, select="topk", chunk_tokens=0, window=0):
    s = make_shape(Q, Q, Q, block_q=block_q, grid=grid, select=select, chunk_tokens=chunk_tokens, window=window)
    return _workspace(lib().sd_rola_workspace_size(ctypes.byref(s), ctypes.byref(lr.p), int(k_keep)), Q.device)


def sd_rola_attention(Q, K, V, g, lr: LowrankParams, k_keep, *, grid, block_q=128, Qn=None, Kn=None,
                      sm_scale=None, out=None, idx_out=None, workspace=None, select="topk", chunk_tokens=0, window=0,
                      stream=None):
    """Fused layer: bf16 O [B, L, H, d]."""
    var = dict(select=select, chunk_tokens=chunk_tokens, window=window)
    torch = _torch()
    B, L, H, d = Q.shape
    if out is None:
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=Q.device)
    if Qn is not None and Qn.stride() != Q.stride():
        raise ValueError("Qn must have the strides of Q")
    if Kn is not None and Kn.stride() != K.stride():
        raise ValueError("Kn must have the strides of K")
    s = make_shape(Q, K, V, out, block_q=block_q, grid=grid, **var)
    ws = workspace if workspace is not None else rola_workspace(Q, lr, k_keep, grid=grid, block_q=block_q, **var)
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)
    gb, gl, gh = _gate_strides(g, B, L, H)
    _check(lib().sd_rola_attention(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qn), _ptr(Kn),
                                   _ptr(g), gb, gl, gh, int(k_keep), float(scale), _ptr(out), _ptr(idx_out), _ptr(ws),
                                   ws.numel(), _stream_ptr(stream)))
    return out


def sd_rola_attention_noalloc(Q, K, V, g, lr: LowrankParams, k_keep, out, *, grid, block_q=128, Qn=None, Kn=None,
                              sm_scale=None, idx_out=None, select="topk", chunk_tokens=0, window=0, stream=None):
    """The fused layer on the library's static device scratch: nothing is
    allocated, here or in the library; `out` (bf16 [B, L, H, d]) is given."""
    B, L, H, d = Q.shape
    if Qn is not None and Qn.stride() != Q.stride():
        raise ValueError("Qn must have the strides of Q")
    if Kn is not None and Kn.stride() != K.stride():
        raise ValueError("Kn must have the strides of K")
    s = make_shape(Q, K, V, out, block_q=block_q, grid=grid, select=select, chunk_tokens=chunk_tokens, window=window)
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)
    gb, gl, gh = _gate_strides(g, B, L, H)
    _check(lib().sd_rola_attention_noalloc(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qn),
                                           _ptr(Kn), _ptr(g), gb, gl, gh, int(k_keep), float(scale), _ptr(out),
                                           _ptr(idx_out), _stream_ptr(stream)))
    return out


def sd_rola_prepare(Q, K, V, lr: LowrankParams, k_keep, workspace, *, grid, block_q=128, Qn=None, Kn=None,
                    idx_out=None, select="topk", chunk_tokens=0, window=0, means=None, stream=None):
    """Phase 1 of the fused layer: block map and low-rank state. means:
    optional (qmean, kmean), the float64 block means sd_qk_norm_rope wrote."""
    s = make_shape(Q, K, V, block_q=block_q, grid=grid, select=select, chunk_tokens=chunk_tokens, window=window)
    qm, km = means if means is not None else (None, None)
    _check(lib().sd_rola_prepare(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qn), _ptr(Kn),
                                 _ptr(qm), _ptr(km), int(k_keep), _ptr(idx_out), _ptr(workspace), workspace.numel(),
                                 _stream_ptr(stream)))


class SavedForward:
    """The forward's O_s (bf16 [B, L, H, d]), RMS ([B, L, H]) and log-sum-exp
    ([B, H, L]) for the backward; allocated for the shape of Q."""

    def __init__(self, Q):
        torch = _torch()
        B, L, H, d = Q.shape
        self.Os = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=Q.device)
        self.rms = torch.empty((B, L, H), dtype=torch.float32, device=Q.device)
        self.lse = torch.empty((B, H, L), dtype=torch.float32, device=Q.device)
        self.s = sd_rola_saved(self.Os.data_ptr(), self.rms.data_ptr(), self.lse.data_ptr())


def sd_rola_apply(Q, K, V, g, lr: LowrankParams, k_keep, workspace, *, grid, block_q=128, Qn=None, sm_scale=None,
                  out=None, idx=None, select="topk", chunk_tokens=0, window=0, save: SavedForward = None,
                  stream=None):
    """Phase 2 of the fused layer: the fused attention kernel; bf16 O. With
    `save`, also keeps O_s, its RMS and the log-sum-exp for the backward
    (sd_rola_apply_save)."""
    torch = _torch()
    B, L, H, d = Q.shape
    if out is None:
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=Q.device)
    s = make_shape(Q, K, V, out, block_q=block_q, grid=grid, select=select, chunk_tokens=chunk_tokens, window=window)
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)
    gb, gl, gh = _gate_strides(g, B, L, H)
    if save is not None:
        _check(lib().sd_rola_apply_save(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qn),
                                        _ptr(g), gb, gl, gh, int(k_keep), float(scale), _ptr(out), _ptr(idx),
                                        _ptr(workspace), workspace.numel(), ctypes.byref(save.s),
                                        _stream_ptr(stream)))
        return out
    _check(lib().sd_rola_apply(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qn), _ptr(g), gb,
                               gl, gh, int(k_keep), float(scale), _ptr(out), _ptr(idx), _ptr(workspace),
                               workspace.numel(), _stream_ptr(stream)))
    return out


def rola_backward_workspace(Q, lr: LowrankParams, k_keep, *, grid, block_q=128, chunk_tokens=0, window=0):
    s = make_shape(Q, Q, Q, block_q=block_q, grid=grid, chunk_tokens=chunk_tokens, window=window)
    return _workspace(lib().sd_rola_backward_workspace_size(ctypes.byref(s), ctypes.byref(lr.p), int(k_keep)),
                      Q.device)


def sd_rola_backward(Q, K, V, g, lr: LowrankParams, k_keep, idx, dO, *, grid, block_q=128, Qn=None, Kn=None,
                     sm_scale=None, want_dP=True, want_dg=True, chunk_tokens=0, window=0, workspace=None,
                     saved: SavedForward = None, stream=None):
    """Gradients of the fused layer for the bf16 output gradient dO (block
    map idx held fixed). Returns a dict of f32 tensors: dQ, dK, dV
    [B, L, H, d]; dQn, dKn (only with Qn / Kn; otherwise that gradient is
    in dQ / dK); dPq, dPk ([rank, d], or [H, rank, d] with per-head
    projections); dg (the shape of g). With `saved` (the forward kept by
    sd_rola_apply(save=...)) the sparse forward is not formed again."""
    torch = _torch()
    B, L, H, d = Q.shape
    s = make_shape(Q, K, V, dO, block_q=block_q, grid=grid, chunk_tokens=chunk_tokens, window=window)
    f32 = dict(dtype=torch.float32, device=Q.device)
    out = {n: torch.empty((B, L, H, d), **f32) for n in ("dQ", "dK", "dV")}
    out["dQn"] = torch.empty((B, L, H, d), **f32) if Qn is not None else None
    out["dKn"] = torch.empty((B, L, H, d), **f32) if Kn is not None else None
    rank = lr.p.rank
    p_shape = (rank, d) if lr.p.P_head_stride == 0 else (H, rank, d)
    out["dPq"] = torch.empty(p_shape, **f32) if want_dP else None
    out["dPk"] = torch.empty(p_shape, **f32) if want_dP else None
    if want_dg:
        out["dg"] = torch.empty_strided(g.shape, g.stride(), **f32)
    else:
        out["dg"] = None
    if workspace is None:
        workspace = rola_backward_workspace(Q, lr, k_keep, grid=grid, block_q=block_q, chunk_tokens=chunk_tokens,
                                            window=window)
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)
    gb, gl, gh = _gate_strides(g, B, L, H)
    _check(lib().sd_rola_backward(ctypes.byref(s), ctypes.byref(lr.p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qn), _ptr(Kn),
                                  _ptr(g), gb, gl, gh, int(k_keep), float(scale), _ptr(idx),
                                  ctypes.byref(saved.s) if saved is not None else None, _ptr(dO),
                                  _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out["dQn"]),
                                  _ptr(out["dKn"]), _ptr(out["dPq"]), _ptr(out["dPk"]), _ptr(out["dg"]),
                                  _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return out
