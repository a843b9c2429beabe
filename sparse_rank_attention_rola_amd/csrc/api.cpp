// libsd C ABI: host-side validation, workspace layout and kernel dispatch.
// Semantics of every entry point are documented in include/sd.h.
#include <algorithm>
#include "sd.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "sd_launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SD_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxL = 131072;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int kMaxArChunks = 4096;

struct Geo {
  int B, H, L, D, bq, bk, Nq, Nk;
  int select;  // SD_SELECT_*
  int ar, win, n_ar;  // causal window: tokens per chunk (L: none), window, chunks
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const sd_attn_shape* s, Geo* g, bool need_grid) {
  if (!s) return fail(SD_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->L < 1) return fail(SD_ERR_INVALID_ARG, "B, H, L must be >= 1");
  if (s->d != 64 && s->d != 128) return fail(SD_ERR_UNSUPPORTED, "d = %d (supported: 64, 128)", s->d);
  if (s->block_q != 64 && s->block_q != 128)
    return fail(SD_ERR_UNSUPPORTED, "block_q = %d (supported: 64, 128)", s->block_q);
  if (s->block_k != 64) return fail(SD_ERR_UNSUPPORTED, "block_k = %d (supported: 64)", s->block_k);
  if (s->L > kMaxL) return fail(SD_ERR_UNSUPPORTED, "L = %d exceeds %d", s->L, kMaxL);
  if (s->select != SD_SELECT_TOPK && s->select != SD_SELECT_FIXED)
    return fail(SD_ERR_INVALID_ARG, "select = %d", s->select);
  if (s->chunk_tokens < 0 || s->window < 0) return fail(SD_ERR_INVALID_ARG, "chunk_tokens and window must be >= 0");
  if (s->chunk_tokens == 0 && s->window != 0) return fail(SD_ERR_INVALID_ARG, "window needs chunk_tokens > 0");
  const int ar = (s->chunk_tokens > 0 && s->chunk_tokens < s->L) ? s->chunk_tokens : s->L;
  if ((s->L + ar - 1) / ar > kMaxArChunks)
    return fail(SD_ERR_UNSUPPORTED, "more than %d autoregressive chunks", kMaxArChunks);
  if (s->select == SD_SELECT_FIXED) need_grid = true;  // the pattern lives on the latent grid
  if (need_grid) {
    if (s->T < 1 || s->Hg < 1 || s->Wg < 1 || (int64_t)s->T * s->Hg * s->Wg != s->L)
      return fail(SD_ERR_INVALID_ARG, "T*Hg*Wg (%d*%d*%d) must equal L = %d", s->T, s->Hg, s->Wg, s->L);
  }
  const int64_t st[12] = {s->sq_b, s->sq_l, s->sq_h, s->sk_b, s->sk_l, s->sk_h,
                          s->sv_b, s->sv_l, s->sv_h, s->so_b, s->so_l, s->so_h};
  for (int i = 0; i < 12; ++i) {
    if (st[i] < 0) return fail(SD_ERR_INVALID_ARG, "negative stride");
    if (st[i] % 8) return fail(SD_ERR_ALIGN, "strides must be multiples of 8 elements (16 bytes)");
  }
  // offsets inside a 64-token tile are 32-bit
  if (std::max(std::max(s->sq_l, s->sk_l), std::max(s->sv_l, s->so_l)) > ((int64_t)1 << 31) / 128)
    return fail(SD_ERR_UNSUPPORTED, "token stride too large");
  // K and V of one (batch, head) are read through 32-bit buffer offsets, and a
  // token row must not overlap the next one
  if (s->sk_l < s->d || s->sv_l < s->d) return fail(SD_ERR_UNSUPPORTED, "K/V token stride smaller than d");
  if ((int64_t)(s->L + 64) * std::max(s->sk_l, s->sv_l) * 2 >= ((int64_t)1 << 32))
    return fail(SD_ERR_UNSUPPORTED, "K/V of one head exceed 4 GiB");
  g->B = s->B;
  g->H = s->H;
  g->L = s->L;
  g->D = s->d;
  g->bq = s->block_q;
  g->bk = s->block_k;
  g->Nq = (s->L + s->block_q - 1) / s->block_q;
  g->Nk = (s->L + s->block_k - 1) / s->block_k;
  g->select = s->select;
  g->ar = ar;
  g->win = s->chunk_tokens > 0 ? s->window : 0;
  g->n_ar = (s->L + ar - 1) / ar;
  if ((int64_t)g->B * g->H * g->Nq >= (int64_t)1 << 31) return fail(SD_ERR_UNSUPPORTED, "too many query blocks");
  if ((int64_t)g->B * g->H > 65535) return fail(SD_ERR_UNSUPPORTED, "B*H exceeds 65535");
  return SD_OK;
}

int check_dev_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(SD_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(SD_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return SD_OK;
}

int check_lowrank(const sd_lowrank_params* lr, const Geo& g) {
  if (!lr) return fail(SD_ERR_INVALID_ARG, "low-rank params are NULL");
  if (lr->rank != 16 && lr->rank != 32) return fail(SD_ERR_UNSUPPORTED, "rank = %d (supported: 16, 32)", lr->rank);
  if (lr->phi != SD_PHI_ELU1) return fail(SD_ERR_UNSUPPORTED, "phi = %d (supported: SD_PHI_ELU1)", lr->phi);
  int rc;
  if ((rc = check_dev_ptr(lr->Pq, "Pq"))) return rc;
  if ((rc = check_dev_ptr(lr->Pk, "Pk"))) return rc;
  if (lr->P_head_stride < 0 || lr->P_head_stride % 8)
    return fail(SD_ERR_ALIGN, "P_head_stride must be a non-negative multiple of 8");
  if (lr->n_rope < 0 || lr->n_rope > sd::kMaxRopePairs || lr->n_rope > lr->rank / 2)
    return fail(SD_ERR_INVALID_ARG, "n_rope = %d out of range", lr->n_rope);
  if (lr->n_rope > 0 && !lr->rope) return fail(SD_ERR_INVALID_ARG, "rope is NULL");
  uint32_t used = 0;
  for (int i = 0; i < lr->n_rope; ++i) {
    const sd_rope_pair& p = lr->rope[i];
    if (p.dim < 0 || p.dim + 1 >= lr->rank || p.axis < 0 || p.axis > 2 || !std::isfinite(p.theta))
      return fail(SD_ERR_INVALID_ARG, "rope pair %d invalid", i);
    const uint32_t bits = 3u << p.dim;
    if (used & bits) return fail(SD_ERR_INVALID_ARG, "rope pairs overlap at pair %d", i);
    used |= bits;
  }
  if (!(lr->rms_eps >= 0.f) || !std::isfinite(lr->rms_eps)) return fail(SD_ERR_INVALID_ARG, "rms_eps invalid");
  if (lr->rms_weight && !aligned(lr->rms_weight, 8)) return fail(SD_ERR_ALIGN, "rms_weight not 8-byte aligned");
  (void)g;
  return SD_OK;
}

// Bump allocator over the caller's workspace (or a size computation when
// base is NULL).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = align_up(off);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

struct SelectWs {
  double* qmean;
  double* kmean;
  double* S;
  uint16_t* khi;  // the key-block means split into bf16 hi + lo (scored selector)
  uint16_t* klo;
  double* knorm2;  // their squared norms
};

// The scored selector forms its scores inside the selection kernel; only the
// fixed pattern keeps a score matrix (one Nq x Nk map for every head).
SelectWs carve_select(Carve& c, const Geo& g) {
  SelectWs w;
  w.qmean = static_cast<double*>(c.take(sizeof(double) * g.B * g.H * g.Nq * g.D));
  w.kmean = static_cast<double*>(c.take(sizeof(double) * g.B * g.H * g.Nk * g.D));
  const size_t s_rows = g.select == SD_SELECT_FIXED ? (size_t)g.Nq : 0;
  w.S = static_cast<double*>(c.take(sizeof(double) * s_rows * g.Nk));
  const size_t split = g.select == SD_SELECT_TOPK ? (size_t)g.B * g.H * g.Nk * g.D : 0;
  w.khi = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * split));
  w.klo = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * split));
  w.knorm2 = static_cast<double*>(c.take(sizeof(double) * (split / g.D)));
  return w;
}

// Runs of 64-token tiles that each write one partial low-rank state: about
// `slots` workgroups in all, `align` tiles a multiple of the run length.
// Each autoregressive chunk gets its own runs (it spans at most
// ceil(ar / 64) + 1 tiles); without a causal window there is one chunk.
sd::RunGeo make_runs(const Geo& g, int64_t slots, int align) {
  const int64_t bh = (int64_t)g.B * g.H;
  const int span = g.n_ar == 1 ? (g.L + 63) / 64 : (g.ar + 63) / 64 + 1;
  const int want = (int)std::min<int64_t>(span, std::max<int64_t>(1, slots / (bh * g.n_ar)));
  int rt = (span + want - 1) / want;
  rt = (rt + align - 1) / align * align;
  sd::RunGeo r;
  r.ar_tokens = g.ar;
  r.run_tiles = rt;
  r.runs_per_ar = (span + rt - 1) / rt;
  r.n_runs = g.n_ar * r.runs_per_ar;
  return r;
}

sd::RunGeo lowrank_runs(const Geo& g) { return make_runs(g, 2048, 1); }

// Runs of the fused prepare pass: at most kPrepareSlots workgroups in all
// where the shape allows it, so that every run is resident at once (three
// 4-wave workgroups per CU on 256 CUs) and none waits for a second round.
// Without a causal window they are aligned to query blocks.
constexpr int64_t kPrepareSlots = 768;
sd::RunGeo prepare_runs(const Geo& g) { return make_runs(g, kPrepareSlots, g.n_ar == 1 ? g.bq / 64 : 1); }

int max_extent(const sd_attn_shape* s) { return std::max(s->T, std::max(s->Hg, s->Wg)); }

struct LowrankWs {
  float2* rope_tab;
  float* partial;
  uint16_t* ct_hi;  // [B*H, n_ar, D, 32]
  uint16_t* ct_lo;
  sd::RunGeo runs;
};

LowrankWs carve_lowrank(Carve& c, const Geo& g, const sd_attn_shape* s, const sd::RunGeo& runs) {
  LowrankWs w;
  w.runs = runs;
  w.rope_tab = static_cast<float2*>(c.take(sizeof(float2) * sd::kMaxRopePairs * max_extent(s)));
  w.partial = static_cast<float*>(c.take(sizeof(float) * g.B * g.H * (size_t)runs.n_runs * 32 * g.D));
  w.ct_hi = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * g.B * g.H * (size_t)g.n_ar * g.D * 32));
  w.ct_lo = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * g.B * g.H * (size_t)g.n_ar * g.D * 32));
  return w;
}

sd::RopeArgs rope_args(const sd_lowrank_params* lr, const sd_attn_shape* s) {
  sd::RopeArgs r{};
  r.n = lr->n_rope;
  r.max_ext = max_extent(s);
  for (int i = 0; i < lr->n_rope; ++i) {
    r.dim[i] = lr->rope[i].dim;
    r.axis[i] = lr->rope[i].axis;
  }
  return r;
}

// Low-rank state: RoPE table, partial C per token chunk, finalisation.
int run_lowrank_state(const sd_attn_shape* s, const Geo& g, const sd_lowrank_params* lr, const void* Kn,
                      const void* V, float* C_out, const LowrankWs& w, hipStream_t st) {
  sd::RopeThetas th{};
  for (int i = 0; i < lr->n_rope; ++i) th.theta[i] = lr->rope[i].theta;
  hipError_t e = sd::launch_rope_table(th, lr->n_rope, max_extent(s), w.rope_tab, st);
  if (e != hipSuccess) return hip_fail(e, "rope table");
  sd::LowrankKvArgs a{};
  a.Kn = static_cast<const uint16_t*>(Kn);
  a.V = static_cast<const uint16_t*>(V);
  a.sk_b = s->sk_b;
  a.sk_l = s->sk_l;
  a.sk_h = s->sk_h;
  a.sv_b = s->sv_b;
  a.sv_l = s->sv_l;
  a.sv_h = s->sv_h;
  a.B = g.B;
  a.H = g.H;
  a.L = g.L;
  a.Hg = s->Hg;
  a.Wg = s->Wg;
  a.runs = w.runs;
  a.Pk = static_cast<const uint16_t*>(lr->Pk);
  a.P_hs = lr->P_head_stride;
  a.rank = lr->rank;
  a.rope_tab = w.rope_tab;
  a.rope = rope_args(lr, s);
  a.partial = w.partial;
  e = sd::launch_lowrank_kv(a, g.D, st);
  if (e != hipSuccess) return hip_fail(e, "low-rank state");
  sd::RankRows rows{};
  for (int r = 0; r < 32; ++r) rows.row[r] = (int8_t)(r < lr->rank ? r : -1);
  e = sd::launch_lowrank_finalize(w.partial, g.B * g.H, w.runs, g.n_ar, g.win, lr->rank, g.D, rows, C_out, w.ct_hi,
                                  w.ct_lo, st);
  if (e != hipSuccess) return hip_fail(e, "low-rank finalize");
  return SD_OK;
}

sd::MapRule map_rule(const Geo& g, int k_keep) {
  sd::MapRule r;
  r.Nq = g.Nq;
  r.bq = g.bq;
  r.bk = g.bk;
  r.L = g.L;
  r.ar_tokens = g.ar;
  r.ar_window = g.win;
  if (g.select == SD_SELECT_FIXED) {  // one map, copied to every (batch, head)
    r.s_rows = g.Nq;
    r.n_rep = g.B * g.H;
    r.rep_stride = (int64_t)g.Nq * k_keep;
  } else {
    r.s_rows = (int64_t)g.B * g.H * g.Nq;
    r.n_rep = 1;
    r.rep_stride = 0;
  }
  return r;
}

// Scores of the selector (block means are ready for SD_SELECT_TOPK), then the
// top-k under the causal window.
int run_scores_topk(const sd_attn_shape* s, const Geo& g, int k_keep, int32_t* idx, const SelectWs& w,
                    hipStream_t st) {
  hipError_t e;
  const sd::MapRule rule = map_rule(g, k_keep);
  if (g.select == SD_SELECT_FIXED) {
    e = sd::launch_fixed_scores(g.L, g.Nq, g.Nk, g.bq, g.bk, s->Hg, s->Wg, w.qmean, w.kmean, w.S, st);
    if (e != hipSuccess) return hip_fail(e, "fixed scores");
    e = sd::launch_topk_rows(w.S, g.Nq, g.Nk, k_keep, rule, idx, st);
  } else {
    e = sd::launch_select_topk(w.qmean, w.kmean, g.B * g.H, g.Nk, g.D, k_keep, rule, w.khi, w.klo, w.knorm2, idx,
                               st);
  }
  if (e != hipSuccess) return hip_fail(e, "top-k");
  return SD_OK;
}

int run_block_select(const sd_attn_shape* s, const Geo& g, const void* Q, const void* K, int k_keep, int32_t* idx,
                     const SelectWs& w, hipStream_t st) {
  if (g.select == SD_SELECT_TOPK) {
    hipError_t e = sd::launch_pool_blocks(static_cast<const uint16_t*>(Q), s->sq_b, s->sq_l, s->sq_h, g.B, g.L, g.H,
                                          g.D, g.bq, w.qmean, st);
    if (e != hipSuccess) return hip_fail(e, "pool Q");
    e = sd::launch_pool_blocks(static_cast<const uint16_t*>(K), s->sk_b, s->sk_l, s->sk_h, g.B, g.L, g.H, g.D, g.bk,
                               w.kmean, st);
    if (e != hipSuccess) return hip_fail(e, "pool K");
  }
  return run_scores_topk(s, g, k_keep, idx, w, st);
}

void fill_attn_common(sd::AttnArgs& a, const sd_attn_shape* s, const Geo& g) {
  a.sq_b = s->sq_b;
  a.sq_l = s->sq_l;
  a.sq_h = s->sq_h;
  a.sk_b = s->sk_b;
  a.sk_l = s->sk_l;
  a.sk_h = s->sk_h;
  a.sv_b = s->sv_b;
  a.sv_l = s->sv_l;
  a.sv_h = s->sv_h;
  a.so_b = s->so_b;
  a.so_l = s->so_l;
  a.so_h = s->so_h;
  a.B = g.B;
  a.H = g.H;
  a.L = g.L;
  a.Nq = g.Nq;
  a.Nk = g.Nk;
  a.Hg = s->Hg;
  a.Wg = s->Wg;
  a.ar_tokens = g.ar;
  a.ar_window = g.win;
}

void fill_attn_lowrank(sd::AttnArgs& a, const sd_lowrank_params* lr, const sd_attn_shape* s, const LowrankWs& w) {
  a.Pq = static_cast<const uint16_t*>(lr->Pq);
  a.P_hs = lr->P_head_stride;
  a.rank = lr->rank;
  a.rope_tab = w.rope_tab;
  a.rope = rope_args(lr, s);
  a.Ct_hi = w.ct_hi;
  a.Ct_lo = w.ct_lo;
  a.eps = lr->rms_eps;
  a.rmsw = static_cast<const uint16_t*>(lr->rms_weight);
}

bool valid_dtype(int dt) { return dt == SD_DTYPE_BF16 || dt == SD_DTYPE_F32; }

}  // namespace

extern "C" {

int sd_keep_count(double sparsity, int n_kblocks) {
  if (n_kblocks < 1 || !(sparsity >= 0.0 && sparsity < 1.0)) return -1;
  const double k = std::ceil((1.0 - sparsity) * n_kblocks - 1e-9);
  return (int)std::min<double>(std::max<double>(k, 1.0), n_kblocks);
}

int sd_rope_default(int rank, double base, sd_rope_pair* out, int max_pairs) {
  if (rank < 2 || !(base > 0.0) || max_pairs < 0 || (max_pairs > 0 && !out)) return -1;
  const int n[3] = {rank - 2 * (rank / 3), rank / 3, rank / 3};
  int cnt = 0, start = 0;
  for (int ax = 0; ax < 3; ++ax) {
    for (int m = 0; m < n[ax] / 2; ++m) {
      if (cnt < max_pairs) {
        out[cnt].dim = start + 2 * m;
        out[cnt].axis = ax;
        out[cnt].theta = (float)std::pow(base, -2.0 * m / n[ax]);
      }
      ++cnt;
    }
    start += n[ax];
  }
  return cnt;
}

size_t sd_block_select_workspace_size(const sd_attn_shape* shape) {
  Geo g;
  if (check_shape(shape, &g, false)) return 0;
  Carve c(nullptr);
  carve_select(c, g);
  return align_up(c.off);
}

int sd_block_select(const sd_attn_shape* shape, const void* Q, const void* K, int k_keep, int32_t* idx, void* ws,
                    size_t ws_bytes, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_shape(shape, &g, false))) return rc;
  if ((rc = check_dev_ptr(Q, "Q")) || (rc = check_dev_ptr(K, "K")) || (rc = check_dev_ptr(idx, "idx", 4)))
    return rc;
  if (k_keep < 1 || k_keep > g.Nk) return fail(SD_ERR_INVALID_ARG, "k_keep = %d not in [1, %d]", k_keep, g.Nk);
  const size_t need = sd_block_select_workspace_size(shape);
  if (!ws || ws_bytes < need) return fail(SD_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(ws, kAlign)) return fail(SD_ERR_ALIGN, "workspace must be 256-byte aligned");
  Carve c(ws);
  const SelectWs w = carve_select(c, g);
  if ((rc = run_block_select(shape, g, Q, K, k_keep, idx, w, static_cast<hipStream_t>(stream)))) return rc;
  return ok();
}

int sd_sparse_attn(const sd_attn_shape* shape, const void* Q, const void* K, const void* V, const int32_t* idx,
                   int k_keep, float sm_scale, void* Os, int os_dtype, float* rms, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_shape(shape, &g, false))) return rc;
  if ((rc = check_dev_ptr(Q, "Q")) || (rc = check_dev_ptr(K, "K")) || (rc = check_dev_ptr(V, "V")) ||
      (rc = check_dev_ptr(idx, "idx", 4)) || (rc = check_dev_ptr(Os, "Os")))
    return rc;
  if (rms && !aligned(rms, 4)) return fail(SD_ERR_ALIGN, "rms misaligned");
  if (k_keep < 1 || k_keep > g.Nk) return fail(SD_ERR_INVALID_ARG, "k_keep = %d not in [1, %d]", k_keep, g.Nk);
  if (!valid_dtype(os_dtype)) return fail(SD_ERR_INVALID_ARG, "os_dtype = %d", os_dtype);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SD_ERR_INVALID_ARG, "sm_scale must be > 0");
  sd::AttnArgs a{};
  fill_attn_common(a, shape, g);
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.Qn = a.Q;
  a.kkeep = k_keep;
  a.idx = idx;
  a.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.out = Os;
  a.out_f32 = os_dtype == SD_DTYPE_F32;
  a.rms = rms;
  const hipError_t e = sd::launch_sparse_attn(a, g.D, g.bq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparse attention");
  return ok();
}

size_t sd_lowrank_workspace_size(const sd_attn_shape* shape, const sd_lowrank_params* lr) {
  Geo g;
  if (check_shape(shape, &g, true)) return 0;
  (void)lr;
  Carve c(nullptr);
  carve_lowrank(c, g, shape, lowrank_runs(g));
  return align_up(c.off);
}

int sd_lowrank_attn(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Qn, const void* Kn,
                    const void* V, void* Olr, int olr_dtype, float* C_out, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_shape(shape, &g, true))) return rc;
  if ((rc = check_lowrank(lr, g))) return rc;
  if ((rc = check_dev_ptr(Qn, "Qn")) || (rc = check_dev_ptr(Kn, "Kn")) || (rc = check_dev_ptr(V, "V")) ||
      (rc = check_dev_ptr(Olr, "Olr")))
    return rc;
  if (C_out && !aligned(C_out, 4)) return fail(SD_ERR_ALIGN, "C_out misaligned");
  if (!valid_dtype(olr_dtype)) return fail(SD_ERR_INVALID_ARG, "olr_dtype = %d", olr_dtype);
  const size_t need = sd_lowrank_workspace_size(shape, lr);
  if (!ws || ws_bytes < need) return fail(SD_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(ws, kAlign)) return fail(SD_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carve c(ws);
  const LowrankWs w = carve_lowrank(c, g, shape, lowrank_runs(g));
  if ((rc = run_lowrank_state(shape, g, lr, Kn, V, C_out, w, st))) return rc;
  sd::AttnArgs a{};
  fill_attn_common(a, shape, g);
  a.Qn = static_cast<const uint16_t*>(Qn);
  a.Q = a.Qn;
  fill_attn_lowrank(a, lr, shape, w);
  a.out = Olr;
  a.out_f32 = olr_dtype == SD_DTYPE_F32;
  const hipError_t e = sd::launch_lowrank_query(a, g.D, g.bq, st);
  if (e != hipSuccess) return hip_fail(e, "low-rank query");
  return ok();
}

int sd_gate_fuse(const sd_attn_shape* shape, const void* Os, const void* Olr, int in_dtype, const float* g_ptr,
                 int64_t g_stride_b, int64_t g_stride_l, int64_t g_stride_h, void* O, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_shape(shape, &g, false))) return rc;
  if ((rc = check_dev_ptr(Os, "Os")) || (rc = check_dev_ptr(Olr, "Olr")) || (rc = check_dev_ptr(O, "O")) ||
      (rc = check_dev_ptr(g_ptr, "g", 4)))
    return rc;
  if (!valid_dtype(in_dtype)) return fail(SD_ERR_INVALID_ARG, "in_dtype = %d", in_dtype);
  if (g_stride_b < 0 || g_stride_l < 0 || g_stride_h < 0) return fail(SD_ERR_INVALID_ARG, "negative gate stride");
  const hipError_t e = sd::launch_gate_fuse(Os, Olr, in_dtype == SD_DTYPE_F32, g_ptr, g_stride_b, g_stride_l,
                                            g_stride_h, O, g.B, g.L, g.H, g.D, shape->so_b, shape->so_l,
                                            shape->so_h, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gate fuse");
  return ok();
}

int sd_quant_fp8_per_token(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                           float* scales, void* stream) {
  if (M < 0 || K < 8) return fail(SD_ERR_INVALID_ARG, "M = %lld, K = %lld", (long long)M, (long long)K);
  if (K % 8 || ldx % 8 || ldq % 8) return fail(SD_ERR_ALIGN, "K, ldx, ldq must be multiples of 8");
  if (K > 16384) return fail(SD_ERR_UNSUPPORTED, "K = %lld exceeds 16384", (long long)K);
  if (ldx < K || ldq < K) return fail(SD_ERR_INVALID_ARG, "ldx and ldq must be >= K");
  if (M > ((int64_t)1 << 31) * 4 - 4) return fail(SD_ERR_UNSUPPORTED, "M too large");
  if (M == 0) return ok();  // nothing to read or write
  int rc;
  if ((rc = check_dev_ptr(x, "x")) || (rc = check_dev_ptr(q, "q", 8)) || (rc = check_dev_ptr(scales, "scales", 4)))
    return rc;
  const hipError_t e = sd::launch_quant_fp8(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, scales,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 quant");
  return ok();
}

int sd_quant_fp8_gate(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                      const void* w_gate, float b_gate, float* g, void* stream) {
  if (M < 0 || K < 8) return fail(SD_ERR_INVALID_ARG, "M = %lld, K = %lld", (long long)M, (long long)K);
  if (K % 8 || ldx % 8 || ldq % 8) return fail(SD_ERR_ALIGN, "K, ldx, ldq must be multiples of 8");
  if (K > 16384) return fail(SD_ERR_UNSUPPORTED, "K = %lld exceeds 16384", (long long)K);
  if (ldx < K || ldq < K) return fail(SD_ERR_INVALID_ARG, "ldx and ldq must be >= K");
  if (!std::isfinite(b_gate)) return fail(SD_ERR_INVALID_ARG, "b_gate must be finite");
  if (M == 0) return ok();  // nothing to read or write
  int rc;
  if ((rc = check_dev_ptr(x, "x")) || (rc = check_dev_ptr(q, "q", 8)) || (rc = check_dev_ptr(scales, "scales", 4)) ||
      (rc = check_dev_ptr(w_gate, "w_gate")) || (rc = check_dev_ptr(g, "g", 4)))
    return rc;
  const hipError_t e = sd::launch_quant_fp8_gate(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, scales,
                                                 static_cast<const uint16_t*>(w_gate), b_gate, g,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 quant + gate");
  return ok();
}

int sd_gemm_fp8_w8a8(const uint8_t* xq, int64_t M, int64_t K, int64_t ldx, const float* sx, const uint8_t* wq,
                     int64_t N, int64_t ldw, const float* sw, void* y, int64_t ldy, void* stream) {
  if (M < 0 || N < 0 || K <= 0)
    return fail(SD_ERR_INVALID_ARG, "M = %lld, N = %lld, K = %lld", (long long)M, (long long)N, (long long)K);
  if (K % 64) return fail(SD_ERR_UNSUPPORTED, "K = %lld is not a multiple of 64", (long long)K);
  if (K > 65536) return fail(SD_ERR_UNSUPPORTED, "K = %lld exceeds 65536", (long long)K);
  if (ldx < K || ldw < K || ldy < N) return fail(SD_ERR_INVALID_ARG, "ldx, ldw must be >= K and ldy >= N");
  if (ldx % 16 || ldw % 16 || ldy % 4) return fail(SD_ERR_ALIGN, "ldx, ldw must be multiples of 16, ldy of 4");
  if (256 * std::max(ldx, ldw) >= ((int64_t)1 << 31))
    return fail(SD_ERR_UNSUPPORTED, "row strides too large for 32-bit tile offsets");
  if (M == 0 || N == 0) return ok();
  int rc;
  if ((rc = check_dev_ptr(xq, "xq")) || (rc = check_dev_ptr(wq, "wq")) || (rc = check_dev_ptr(sx, "sx", 4)) ||
      (rc = check_dev_ptr(sw, "sw")) || (rc = check_dev_ptr(y, "y", 8)))
    return rc;
  sd::GemmFp8Args a{xq, wq, sx, sw, static_cast<uint16_t*>(y), M, N, K, ldx, ldw, ldy};
  const hipError_t e = sd::launch_gemm_fp8(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 gemm");
  return ok();
}

int sd_qk_norm_rope(int B, int L, int H, int d, int T, int Hg, int Wg, const void* q, const void* k,
                    int64_t ld_in, const void* gamma_q, const void* gamma_k, float eps, const sd_rope_pair* rope,
                    int n_rope, void* Q, void* K, void* Qn, void* Kn, double* qmean, double* kmean, int block_q,
                    int block_k, void* stream) {
  if (B < 1 || L < 1 || H < 1) return fail(SD_ERR_INVALID_ARG, "B, L, H must be >= 1");
  if (d != 64 && d != 128) return fail(SD_ERR_UNSUPPORTED, "d = %d (supported: 64, 128)", d);
  if ((int64_t)H * d > 8192) return fail(SD_ERR_UNSUPPORTED, "H*d = %d exceeds 8192", H * d);
  if (T < 1 || Hg < 1 || Wg < 1 || (int64_t)T * Hg * Wg != L)
    return fail(SD_ERR_INVALID_ARG, "T*Hg*Wg (%d*%d*%d) must equal L = %d", T, Hg, Wg, L);
  if (ld_in < (int64_t)H * d) return fail(SD_ERR_INVALID_ARG, "ld_in must be >= H*d");
  if (ld_in % 8) return fail(SD_ERR_ALIGN, "ld_in must be a multiple of 8");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(SD_ERR_INVALID_ARG, "eps invalid");
  if (n_rope < 0 || n_rope > d / 2) return fail(SD_ERR_INVALID_ARG, "n_rope = %d out of range", n_rope);
  if (n_rope > 0 && !rope) return fail(SD_ERR_INVALID_ARG, "rope is NULL");
  sd::QkNormRopeArgs a{};
  for (int i = 0; i < sd::kQkMaxPairs; ++i) {
    a.pair_axis[i] = -1;
    a.pair_theta[i] = 0.f;
  }
  for (int i = 0; i < n_rope; ++i) {
    const sd_rope_pair& p = rope[i];
    if (p.dim < 0 || p.dim + 1 >= d || p.dim % 2 || p.axis < 0 || p.axis > 2 || !std::isfinite(p.theta))
      return fail(SD_ERR_INVALID_ARG, "rope pair %d invalid (dims must be even, inside the head)", i);
    if (a.pair_axis[p.dim / 2] >= 0) return fail(SD_ERR_INVALID_ARG, "rope pairs overlap at pair %d", i);
    a.pair_axis[p.dim / 2] = (int8_t)p.axis;
    a.pair_theta[p.dim / 2] = p.theta;
  }
  int rc;
  if ((rc = check_dev_ptr(q, "q")) || (rc = check_dev_ptr(k, "k")) || (rc = check_dev_ptr(Q, "Q")) ||
      (rc = check_dev_ptr(K, "K")) || (rc = check_dev_ptr(Qn, "Qn")) || (rc = check_dev_ptr(Kn, "Kn")))
    return rc;
  if ((gamma_q && !aligned(gamma_q, 16)) || (gamma_k && !aligned(gamma_k, 16)))
    return fail(SD_ERR_ALIGN, "gamma must be 16-byte aligned");
  if (qmean || kmean) {
    if ((block_q != 64 && block_q != 128) || block_k != 64)
      return fail(SD_ERR_UNSUPPORTED, "block means need block_q in {64, 128} and block_k = 64");
    if ((qmean && !aligned(qmean, 8)) || (kmean && !aligned(kmean, 8)))
      return fail(SD_ERR_ALIGN, "block means must be 8-byte aligned");
  }
  a.qmean = qmean;
  a.kmean = kmean;
  a.block_q = block_q;
  a.block_k = block_k;
  a.rcp_block_q = 1.0 / block_q;
  a.rcp_block_k = 1.0 / block_k;
  a.seg_rows = 128;  // a multiple of both block sizes
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.ld_in = ld_in;
  a.gamma_q = static_cast<const uint16_t*>(gamma_q);
  a.gamma_k = static_cast<const uint16_t*>(gamma_k);
  a.eps = eps;
  a.B = B;
  a.L = L;
  a.H = H;
  a.d = d;
  a.Hg = Hg;
  a.Wg = Wg;
  a.Q = static_cast<uint16_t*>(Q);
  a.K = static_cast<uint16_t*>(K);
  a.Qn = static_cast<uint16_t*>(Qn);
  a.Kn = static_cast<uint16_t*>(Kn);
  const hipError_t e = sd::launch_qk_norm_rope(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "q/k norm + rope");
  return ok();
}

}  // extern "C"

namespace {

struct RolaWs {
  SelectWs sel;
  int32_t* idx;
  LowrankWs lr;
  size_t bytes;
};

// Workspace of the fused entry points (sizes only when ws is NULL).
RolaWs carve_rola(void* ws, const Geo& g, const sd_attn_shape* shape, int k_keep) {
  Carve c(ws);
  RolaWs w;
  w.sel = carve_select(c, g);
  w.idx = static_cast<int32_t*>(c.take(sizeof(int32_t) * g.B * g.H * (size_t)g.Nq * k_keep));
  // the fused pass writes one partial state per run of tiles
  w.lr = carve_lowrank(c, g, shape, prepare_runs(g));
  w.bytes = align_up(c.off);
  return w;
}

}  // namespace

extern "C" {

size_t sd_rola_workspace_size(const sd_attn_shape* shape, const sd_lowrank_params* lr, int k_keep) {
  Geo g;
  if (check_shape(shape, &g, true)) return 0;
  if (k_keep < 1 || k_keep > g.Nk) return 0;
  (void)lr;
  return carve_rola(nullptr, g, shape, k_keep).bytes;
}

}  // extern "C"

namespace {

// Validation shared by the fused entry points.
// Everything but the workspace.
int check_rola_args(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                    const void* V, const void* Qn, const void* Kn, int k_keep, const void* idx, Geo* g) {
  int rc;
  if ((rc = check_shape(shape, g, true))) return rc;
  if ((rc = check_lowrank(lr, *g))) return rc;
  if ((rc = check_dev_ptr(Q, "Q")) || (rc = check_dev_ptr(K, "K")) || (rc = check_dev_ptr(V, "V"))) return rc;
  if (Qn && (rc = check_dev_ptr(Qn, "Qn"))) return rc;
  if (Kn && (rc = check_dev_ptr(Kn, "Kn"))) return rc;
  if (idx && !aligned(idx, 4)) return fail(SD_ERR_ALIGN, "block map pointer misaligned");
  if (k_keep < 1 || k_keep > g->Nk) return fail(SD_ERR_INVALID_ARG, "k_keep = %d not in [1, %d]", k_keep, g->Nk);
  return SD_OK;
}

int check_rola(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K, const void* V,
               const void* Qn, const void* Kn, int k_keep, const void* idx, size_t ws_bytes, const void* ws,
               Geo* g) {
  int rc;
  if ((rc = check_rola_args(shape, lr, Q, K, V, Qn, Kn, k_keep, idx, g))) return rc;
  const size_t need = sd_rola_workspace_size(shape, lr, k_keep);
  if (!ws || ws_bytes < need) return fail(SD_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(ws, kAlign)) return fail(SD_ERR_ALIGN, "workspace must be 256-byte aligned");
  return SD_OK;
}

int check_apply_extra(const void* O, const float* g_ptr, float sm_scale, int64_t gb, int64_t gl, int64_t gh) {
  int rc;
  if ((rc = check_dev_ptr(O, "O")) || (rc = check_dev_ptr(g_ptr, "g", 4))) return rc;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SD_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (gb < 0 || gl < 0 || gh < 0) return fail(SD_ERR_INVALID_ARG, "negative gate stride");
  return SD_OK;
}

// Arguments of the stream pass (the low-rank state of every run of tiles)
// and the rank row of each of its slots.
sd::PrepareArgs prepare_args(const sd_attn_shape* s, const Geo& g, const sd_lowrank_params* lr, const void* Q,
                             const void* K, const void* V, const void* Kn, const LowrankWs& w, sd::RankRows* rows) {
  sd::PrepareArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.Kn = static_cast<const uint16_t*>(Kn ? Kn : K);
  a.V = static_cast<const uint16_t*>(V);
  a.sq_b = s->sq_b;
  a.sq_l = s->sq_l;
  a.sq_h = s->sq_h;
  a.sk_b = s->sk_b;
  a.sk_l = s->sk_l;
  a.sk_h = s->sk_h;
  a.sv_b = s->sv_b;
  a.sv_l = s->sv_l;
  a.sv_h = s->sv_h;
  a.B = g.B;
  a.H = g.H;
  a.L = g.L;
  a.Nq = g.Nq;
  a.Nk = g.Nk;
  a.block_q = g.bq;
  a.Hg = s->Hg;
  a.Wg = s->Wg;
  a.rcp_hw = 1.0f / (float)(s->Hg * s->Wg);
  a.rcp_wg = 1.0f / (float)s->Wg;
  a.runs = w.runs;
  a.Pk = static_cast<const uint16_t*>(lr->Pk);
  a.P_hs = lr->P_head_stride;
  a.rank = lr->rank;
  a.rope_tab = w.rope_tab;
  a.rope = rope_args(lr, s);
  // rank slots: each RoPE pair takes the next two slots, then each rank
  // outside every pair one slot; the rest stay empty
  for (int r = 0; r < 32; ++r) rows->row[r] = -1;
  for (int i = 0; i < 32; ++i) a.slot_rank[i] = -1;
  for (int p = 0; p < 16; ++p) a.slot_pair[p] = -1;
  int nslot = 0;
  for (int m = 0; m < lr->n_rope; ++m) {
    a.slot_pair[nslot / 2] = (int8_t)m;
    for (int k = 0; k < 2; ++k) {
      a.slot_rank[nslot] = (int8_t)(lr->rope[m].dim + k);
      rows->row[lr->rope[m].dim + k] = (int8_t)nslot;
      ++nslot;
    }
  }
  for (int r = 0; r < lr->rank; ++r)
    if (rows->row[r] < 0) {
      a.slot_rank[nslot] = (int8_t)r;
      rows->row[r] = (int8_t)nslot;
      ++nslot;
    }
  a.slot_mask = 0;
  for (int i = 0; i < 32; ++i)
    if (a.slot_rank[i] >= 0) a.slot_mask |= 1u << i;
  a.kmean = nullptr;
  a.partial = w.partial;
  return a;
}

// A second stream per device for the prepare phase: its HBM-bound stream
// pass over K and V runs there beside the ALU-bound block selection on the
// caller's stream. Events fork it from the caller's stream (it starts after
// everything enqueued there before) and join it back (the caller's later work
// waits for it), so to the caller the call stays ordered on its own stream,
// also under graph capture. The streams and events live until the process
// ends; a mutex serialises the fork/join sequences of host threads.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

std::mutex g_side_mu;

int side_stream(SideStream** out) {
  static std::vector<SideStream> per_dev;
  int dev = 0, n = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_fail(e, "side stream: device");
  if ((int)per_dev.size() < n) per_dev.resize(n);
  SideStream& ss = per_dev[dev];
  if (!ss.s) {
    if ((e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "side stream: create");
  }
  *out = &ss;
  return SD_OK;
}

int run_rope_table(const sd_attn_shape* s, const sd_lowrank_params* lr, float2* tab, hipStream_t st) {
  sd::RopeThetas th{};
  for (int i = 0; i < lr->n_rope; ++i) th.theta[i] = lr->rope[i].theta;
  const hipError_t e = sd::launch_rope_table(th, lr->n_rope, max_extent(s), tab, st);
  if (e != hipSuccess) return hip_fail(e, "rope table");
  return SD_OK;
}

// Block map and low-rank state: a stream pass over K (Kn) and V for the
// partial states and their sum, and the block selection (pooling, score
// GEMM, top-k, or the fixed pattern).
// When the stream pass reads K itself and its runs are whole key blocks (no
// causal window), it also forms the key-block means; everything then runs in
// order on the caller's stream (the Q pooling beside the stream pass would
// only share HBM with it), as it does on a stream being captured into a
// graph (and when the caller asks for no side stream). Otherwise the
// selection, which keeps the vector ALUs busy, runs on the caller's stream
// beside the HBM-bound stream pass on the side stream.
// sel_given: the selection workspace with the caller's block means of Q and
// K (the q/k producer wrote them), so nothing pools them here.
int run_prepare(const sd_attn_shape* s, const Geo& g, const sd_lowrank_params* lr, const void* Q, const void* K,
                const void* V, const void* Kn, int k_keep, int32_t* idx, const RolaWs& w, hipStream_t st,
                bool allow_side = true, const SelectWs* sel_given = nullptr) {
  int rc = run_rope_table(s, lr, w.lr.rope_tab, st);
  if (rc) return rc;
  sd::RankRows rows;
  sd::PrepareArgs a = prepare_args(s, g, lr, Q, K, V, Kn, w.lr, &rows);
  const bool scored = g.select == SD_SELECT_TOPK;
  const bool pool = scored && !sel_given;
  const SelectWs& sel = sel_given ? *sel_given : w.sel;
  const bool k_in_stream = pool && a.Kn == a.K && g.n_ar == 1;
  a.kmean = k_in_stream ? w.sel.kmean : nullptr;
  hipError_t e;
  auto stream_pass = [&](hipStream_t on) -> int {
    hipError_t e2 = sd::launch_prepare_stream(a, g.D, on);
    if (e2 != hipSuccess) return hip_fail(e2, "prepare pass");
    e2 = sd::launch_lowrank_finalize(w.lr.partial, g.B * g.H, w.lr.runs, g.n_ar, g.win, lr->rank, g.D, rows, nullptr,
                                     w.lr.ct_hi, w.lr.ct_lo, on);
    if (e2 != hipSuccess) return hip_fail(e2, "low-rank finalize");
    return SD_OK;
  };
  // A stream being captured into a graph keeps everything on itself: the
  // side stream is shared by the host threads, and forking it into one
  // thread's capture would pull another thread's eager work into that graph.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if ((e = hipStreamIsCapturing(st, &cap)) != hipSuccess) return hip_fail(e, "prepare: capture status");
  if (k_in_stream || cap != hipStreamCaptureStatusNone || !allow_side) {
    if (pool) {
      e = sd::launch_pool_blocks(a.Q, s->sq_b, s->sq_l, s->sq_h, g.B, g.L, g.H, g.D, g.bq, w.sel.qmean, st);
      if (e == hipSuccess && !k_in_stream)
        e = sd::launch_pool_blocks(a.K, s->sk_b, s->sk_l, s->sk_h, g.B, g.L, g.H, g.D, g.bk, w.sel.kmean, st);
      if (e != hipSuccess) return hip_fail(e, "block pooling");
    }
    if ((rc = stream_pass(st))) return rc;
    return run_scores_topk(s, g, k_keep, idx, sel, st);
  }
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = nullptr;
  if ((rc = side_stream(&side))) return rc;
  e = hipEventRecord(side->fork, st);
  if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
  if (e != hipSuccess) return hip_fail(e, "prepare: fork");
  rc = stream_pass(side->s);
  e = hipEventRecord(side->join, side->s);
  if (rc || e != hipSuccess) {
    // a failed launch still joins, so that no fork is left open and the side
    // stream's work is ordered before whatever the caller enqueues next
    if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
    if (rc) return rc;
    return hip_fail(e, "prepare: join");
  }
  if (pool) {
    e = sd::launch_pool_blocks(a.Q, s->sq_b, s->sq_l, s->sq_h, g.B, g.L, g.H, g.D, g.bq, w.sel.qmean, st);
    if (e == hipSuccess)
      e = sd::launch_pool_blocks(a.K, s->sk_b, s->sk_l, s->sk_h, g.B, g.L, g.H, g.D, g.bk, w.sel.kmean, st);
  }
  rc = e == hipSuccess ? run_scores_topk(s, g, k_keep, idx, sel, st) : hip_fail(e, "block pooling");
  // the join comes after a failed launch too
  e = hipStreamWaitEvent(st, side->join, 0);
  if (rc) return rc;
  if (e != hipSuccess) return hip_fail(e, "prepare: join");
  return SD_OK;
}

int run_apply(const sd_attn_shape* shape, const Geo& g, const sd_lowrank_params* lr, const void* Q, const void* K,
              const void* V, const void* Qn, const float* g_ptr, int64_t gb, int64_t gl, int64_t gh, int k_keep,
              float sm_scale, void* O, const int32_t* idx, const RolaWs& w, hipStream_t st,
              const sd_rola_saved* save = nullptr) {
  sd::AttnArgs a{};
  fill_attn_common(a, shape, g);
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.Qn = static_cast<const uint16_t*>(Qn ? Qn : Q);
  a.kkeep = k_keep;
  a.idx = idx;
  a.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  fill_attn_lowrank(a, lr, shape, w.lr);
  a.out = O;
  a.out_f32 = 0;
  a.g = g_ptr;
  a.g_sb = gb;
  a.g_sl = gl;
  a.g_sh = gh;
  if (save) {
    a.os_save = static_cast<uint16_t*>(save->Os);
    a.rms = save->rms;
    a.lse = save->lse;
  }
  const hipError_t e = sd::launch_rola_fused(a, g.D, g.bq, st);
  if (e != hipSuccess) return hip_fail(e, "fused attention");
  return SD_OK;
}

}  // namespace

extern "C" {

int sd_rola_prepare(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                    const void* V, const void* Qn, const void* Kn, const double* qmean, const double* kmean,
                    int k_keep, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_rola(shape, lr, Q, K, V, Qn, Kn, k_keep, idx_out, ws_bytes, ws, &g))) return rc;
  if ((qmean == nullptr) != (kmean == nullptr)) return fail(SD_ERR_INVALID_ARG, "give both block means or neither");
  if ((qmean && !aligned(qmean, 8)) || (kmean && !aligned(kmean, 8)))
    return fail(SD_ERR_ALIGN, "block means must be 8-byte aligned");
  const RolaWs w = carve_rola(ws, g, shape, k_keep);
  SelectWs given = w.sel;
  given.qmean = const_cast<double*>(qmean);
  given.kmean = const_cast<double*>(kmean);
  if ((rc = run_prepare(shape, g, lr, Q, K, V, Kn, k_keep, idx_out ? idx_out : w.idx, w,
                        static_cast<hipStream_t>(stream), true, qmean ? &given : nullptr)))
    return rc;
  return ok();
}

int sd_rola_apply(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                  const void* V, const void* Qn, const float* g_ptr, int64_t g_stride_b, int64_t g_stride_l,
                  int64_t g_stride_h, int k_keep, float sm_scale, void* O, const int32_t* idx, void* ws,
                  size_t ws_bytes, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_rola(shape, lr, Q, K, V, Qn, nullptr, k_keep, idx, ws_bytes, ws, &g))) return rc;
  if ((rc = check_apply_extra(O, g_ptr, sm_scale, g_stride_b, g_stride_l, g_stride_h))) return rc;
  const RolaWs w = carve_rola(ws, g, shape, k_keep);
  if ((rc = run_apply(shape, g, lr, Q, K, V, Qn, g_ptr, g_stride_b, g_stride_l, g_stride_h, k_keep, sm_scale, O,
                      idx ? idx : w.idx, w, static_cast<hipStream_t>(stream))))
    return rc;
  return ok();
}

// The gate's (b, l, h) strides address every stored element from one index
// of its non-broadcast dimensions: sorted by stride, each dimension of
// extent > 1 and stride > 0 steps past the whole span of the smaller ones.
// (A stride of 0 is a broadcast; the gradient then sums over it.)
static bool gate_strides_disjoint(const Geo& g, int64_t sb, int64_t sl, int64_t sh) {
  std::vector<std::pair<int64_t, int64_t>> dims;  // (stride, extent)
  if (sb > 0 && g.B > 1) dims.push_back({sb, g.B});
  if (sl > 0 && g.L > 1) dims.push_back({sl, g.L});
  if (sh > 0 && g.H > 1) dims.push_back({sh, g.H});
  std::sort(dims.begin(), dims.end());
  int64_t span = 1;
  for (const auto& d : dims) {
    if (d.first < span) return false;
    span = d.first * d.second;
  }
  return true;
}

int check_saved(const sd_rola_saved* sv) {
  if (!sv) return fail(SD_ERR_INVALID_ARG, "saved-forward struct is NULL");
  int rc;
  if ((rc = check_dev_ptr(sv->Os, "saved Os", 8)) || (rc = check_dev_ptr(sv->rms, "saved rms", 4)) ||
      (rc = check_dev_ptr(sv->lse, "saved lse", 4)))
    return rc;
  return SD_OK;
}

int sd_rola_apply_save(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                       const void* V, const void* Qn, const float* g_ptr, int64_t g_stride_b, int64_t g_stride_l,
                       int64_t g_stride_h, int k_keep, float sm_scale, void* O, const int32_t* idx, void* ws,
                       size_t ws_bytes, const sd_rola_saved* save, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_rola(shape, lr, Q, K, V, Qn, nullptr, k_keep, idx, ws_bytes, ws, &g))) return rc;
  if ((rc = check_apply_extra(O, g_ptr, sm_scale, g_stride_b, g_stride_l, g_stride_h))) return rc;
  if ((rc = check_saved(save))) return rc;
  const RolaWs w = carve_rola(ws, g, shape, k_keep);
  if ((rc = run_apply(shape, g, lr, Q, K, V, Qn, g_ptr, g_stride_b, g_stride_l, g_stride_h, k_keep, sm_scale, O,
                      idx ? idx : w.idx, w, static_cast<hipStream_t>(stream), save)))
    return rc;
  return ok();
}

int sd_rola_attention(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                      const void* V, const void* Qn, const void* Kn, const float* g_ptr, int64_t g_stride_b,
                      int64_t g_stride_l, int64_t g_stride_h, int k_keep, float sm_scale, void* O, int32_t* idx_out,
                      void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_rola(shape, lr, Q, K, V, Qn, Kn, k_keep, idx_out, ws_bytes, ws, &g))) return rc;
  if ((rc = check_apply_extra(O, g_ptr, sm_scale, g_stride_b, g_stride_l, g_stride_h))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RolaWs w = carve_rola(ws, g, shape, k_keep);
  int32_t* idx = idx_out ? idx_out : w.idx;
  if ((rc = run_prepare(shape, g, lr, Q, K, V, Kn, k_keep, idx, w, st))) return rc;
  if ((rc = run_apply(shape, g, lr, Q, K, V, Qn, g_ptr, g_stride_b, g_stride_l, g_stride_h, k_keep, sm_scale, O, idx,
                      w, st)))
    return rc;
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The fused layer without a caller workspace, for callers that cannot
// allocate: its scratch is a static device array of SD_NOALLOC_SCRATCH_BYTES
// that every GPU the library runs on holds until the process ends. Host code
// reaches a device's copy only through the address hipGetSymbolAddress
// returns for that device (kept per device, taken once with the device
// current); the array's own name is a host-side stand-in.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;

int scratch_address(void** out) {
  static std::vector<void*> per_dev;
  int dev = 0, n = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_fail(e, "static scratch: device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)per_dev.size() < n) per_dev.resize(n, nullptr);
  if (!per_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "static scratch: symbol address");
    per_dev[dev] = ptr;
  }
  *out = per_dev[dev];
  return SD_OK;
}

}  // namespace

extern "C" {

int sd_rola_attention_noalloc(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                              const void* V, const void* Qn, const void* Kn, const float* g_ptr, int64_t g_stride_b,
                              int64_t g_stride_l, int64_t g_stride_h, int k_keep, float sm_scale, void* O,
                              int32_t* idx_out, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_rola_args(shape, lr, Q, K, V, Qn, Kn, k_keep, idx_out, &g))) return rc;
  if ((rc = check_apply_extra(O, g_ptr, sm_scale, g_stride_b, g_stride_l, g_stride_h))) return rc;
  const size_t need = sd_rola_workspace_size(shape, lr, k_keep);
  if (need > (size_t)SD_NOALLOC_SCRATCH_BYTES)
    return fail(SD_ERR_UNSUPPORTED, "this shape needs %zu bytes of scratch; the static buffer holds %zu", need,
                (size_t)SD_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const RolaWs w = carve_rola(ws, g, shape, k_keep);
  int32_t* idx = idx_out ? idx_out : w.idx;
  // no side stream: the prepare phase runs in order on the caller's stream
  if ((rc = run_prepare(shape, g, lr, Q, K, V, Kn, k_keep, idx, w, st, false))) return rc;
  if ((rc = run_apply(shape, g, lr, Q, K, V, Qn, g_ptr, g_stride_b, g_stride_l, g_stride_h, k_keep, sm_scale, O, idx,
                      w, st)))
    return rc;
  return ok();
}

}  // extern "C"

namespace {

// Workspace of the backward (sizes only when ws is NULL).
struct BwdWs {
  LowrankWs lr;
  float* C;  // [B*H, n_ar, rank, D]
  float *rms, *lse, *Dd, *dg_head, *qt, *dy, *da, *db, *dQn_tmp;
  uint16_t *Os, *dOs;
  float* dC_part;
  sd::RunGeo dC_runs;
  float* dC;
  uint16_t *dCt_hi, *dCt_lo;
  float* dP_part;
  sd::RunGeo dP_runs;
  int32_t *tlist, *toff, *korder;
  size_t bytes;
};

BwdWs carve_bwd(void* ws, const Geo& g, const sd_attn_shape* shape, const sd_lowrank_params* lr, int k_keep) {
  Carve c(ws);
  BwdWs w;
  const size_t BH = (size_t)g.B * g.H, rows = BH * g.L;
  w.lr = carve_lowrank(c, g, shape, prepare_runs(g));
  w.C = static_cast<float*>(c.take(sizeof(float) * BH * g.n_ar * 32 * g.D));
  w.Os = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * rows * g.D));
  w.rms = static_cast<float*>(c.take(sizeof(float) * rows));
  w.lse = static_cast<float*>(c.take(sizeof(float) * rows));
  w.Dd = static_cast<float*>(c.take(sizeof(float) * rows));
  w.dg_head = static_cast<float*>(c.take(sizeof(float) * rows));
  w.qt = static_cast<float*>(c.take(sizeof(float) * rows * 32));
  w.dy = static_cast<float*>(c.take(sizeof(float) * rows * g.D));
  w.da = static_cast<float*>(c.take(sizeof(float) * rows * 32));
  w.db = static_cast<float*>(c.take(sizeof(float) * rows * 32));
  w.dQn_tmp = static_cast<float*>(c.take(sizeof(float) * rows * g.D));
  w.dOs = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * rows * g.D));
  w.dC_runs = make_runs(g, kPrepareSlots, 1);
  w.dC_part = static_cast<float*>(c.take(sizeof(float) * BH * w.dC_runs.n_runs * 32 * g.D));
  w.dC = static_cast<float*>(c.take(sizeof(float) * BH * g.n_ar * 32 * g.D));
  w.dCt_hi = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * BH * g.n_ar * g.D * 32));
  w.dCt_lo = static_cast<uint16_t*>(c.take(sizeof(uint16_t) * BH * g.n_ar * g.D * 32));
  Geo whole = g;  // one run set over the whole sequence for the projection gradients
  whole.n_ar = 1;
  whole.ar = g.L;
  w.dP_runs = make_runs(whole, kPrepareSlots, 1);
  w.dP_part = static_cast<float*>(c.take(sizeof(float) * BH * w.dP_runs.n_runs * 32 * g.D));
  w.tlist = static_cast<int32_t*>(c.take(sizeof(int32_t) * BH * g.Nq * (size_t)k_keep));
  w.toff = static_cast<int32_t*>(c.take(sizeof(int32_t) * BH * (g.Nk + 1)));
  w.korder = static_cast<int32_t*>(c.take(sizeof(int32_t) * BH * g.Nk));
  (void)lr;
  w.bytes = align_up(c.off);
  return w;
}

}  // namespace

extern "C" {

size_t sd_rola_backward_workspace_size(const sd_attn_shape* shape, const sd_lowrank_params* lr, int k_keep) {
  Geo g;
  if (check_shape(shape, &g, true)) return 0;
  if (k_keep < 1 || k_keep > g.Nk) return 0;
  return carve_bwd(nullptr, g, shape, lr, k_keep).bytes;
}

int sd_rola_backward(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                     const void* V, const void* Qn, const void* Kn, const float* g_ptr, int64_t g_stride_b,
                     int64_t g_stride_l, int64_t g_stride_h, int k_keep, float sm_scale, const int32_t* idx,
                     const sd_rola_saved* saved, const void* dO, float* dQ, float* dK, float* dV, float* dQn,
                     float* dKn, float* dPq, float* dPk, float* dg, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  int rc;
  if ((rc = check_shape(shape, &g, true))) return rc;
  if ((rc = check_lowrank(lr, g))) return rc;
  if ((rc = check_dev_ptr(Q, "Q")) || (rc = check_dev_ptr(K, "K")) || (rc = check_dev_ptr(V, "V")) ||
      (rc = check_dev_ptr(idx, "idx", 4)) || (rc = check_dev_ptr(dO, "dO")) || (rc = check_dev_ptr(dQ, "dQ")) ||
      (rc = check_dev_ptr(dK, "dK")) || (rc = check_dev_ptr(dV, "dV")))
    return rc;
  if ((rc = check_apply_extra(dO, g_ptr, sm_scale, g_stride_b, g_stride_l, g_stride_h))) return rc;
  if (Qn && (rc = check_dev_ptr(Qn, "Qn"))) return rc;
  if (Kn && (rc = check_dev_ptr(Kn, "Kn"))) return rc;
  if ((Qn != nullptr) != (dQn != nullptr)) return fail(SD_ERR_INVALID_ARG, "dQn must be given exactly when Qn is");
  if ((Kn != nullptr) != (dKn != nullptr)) return fail(SD_ERR_INVALID_ARG, "dKn must be given exactly when Kn is");
  if ((dQn && !aligned(dQn, 16)) || (dKn && !aligned(dKn, 16))) return fail(SD_ERR_ALIGN, "dQn / dKn misaligned");
  if ((dPq && !aligned(dPq, 4)) || (dPk && !aligned(dPk, 4)) || (dg && !aligned(dg, 4)))
    return fail(SD_ERR_ALIGN, "dPq / dPk / dg misaligned");
  if (dg && !gate_strides_disjoint(g, g_stride_b, g_stride_l, g_stride_h))
    return fail(SD_ERR_UNSUPPORTED, "gate strides overlap: dg elements would be written by several (b, l, h)");
  if (k_keep < 1 || k_keep > g.Nk) return fail(SD_ERR_INVALID_ARG, "k_keep = %d not in [1, %d]", k_keep, g.Nk);
  if (saved && (rc = check_saved(saved))) return rc;
  // the staged dO_s tiles are read through 32-bit buffer offsets
  if ((int64_t)(g.L + 64) * std::max<int64_t>((int64_t)g.H * g.D, shape->sq_l) * 2 >= ((int64_t)1 << 32))
    return fail(SD_ERR_UNSUPPORTED, "L * H * d (or Q's token stride) too large for the backward");
  const size_t need = sd_rola_backward_workspace_size(shape, lr, k_keep);
  if (!ws || ws_bytes < need) return fail(SD_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(ws, kAlign)) return fail(SD_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const BwdWs w = carve_bwd(ws, g, shape, lr, k_keep);
  const int BH = g.B * g.H;
  const int64_t rows = (int64_t)BH * g.L;

  // forward recomputation: the low-rank state (rows and transposed hi / lo)
  if ((rc = run_rope_table(shape, lr, w.lr.rope_tab, st))) return rc;
  sd::RankRows rrows;
  const sd::PrepareArgs pa = prepare_args(shape, g, lr, Q, K, V, Kn, w.lr, &rrows);
  hipError_t e = sd::launch_prepare_stream(pa, g.D, st);
  if (e != hipSuccess) return hip_fail(e, "state pass");
  e = sd::launch_lowrank_finalize(w.lr.partial, BH, w.lr.runs, g.n_ar, g.win, lr->rank, g.D, rrows, w.C, w.lr.ct_hi,
                                  w.lr.ct_lo, st);
  if (e != hipSuccess) return hip_fail(e, "state finalize");
  // the sparse branch output O_s (bf16), its RMS and log-sum-exp: kept by
  // the forward, or formed here by the sparse kernel
  const uint16_t* Os = saved ? static_cast<const uint16_t*>(saved->Os) : w.Os;
  const float* rms = saved ? saved->rms : w.rms;
  const float* lse = saved ? saved->lse : w.lse;
  if (!saved) {
    sd::AttnArgs a{};
    fill_attn_common(a, shape, g);
    a.so_b = (int64_t)g.L * g.H * g.D;
    a.so_l = (int64_t)g.H * g.D;
    a.so_h = g.D;
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.V = static_cast<const uint16_t*>(V);
    a.Qn = a.Q;
    a.kkeep = k_keep;
    a.idx = idx;
    a.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
    a.out = w.Os;
    a.out_f32 = 0;
    a.rms = w.rms;
    a.lse = w.lse;
    e = sd::launch_sparse_attn(a, g.D, g.bq, st);
    if (e != hipSuccess) return hip_fail(e, "sparse forward");
  }
  sd::BwdArgs b{};
  b.B = g.B;
  b.H = g.H;
  b.L = g.L;
  b.Nq = g.Nq;
  b.Nk = g.Nk;
  b.kkeep = k_keep;
  b.Hg = shape->Hg;
  b.Wg = shape->Wg;
  b.block_q = g.bq;
  b.ar_tokens = g.ar;
  b.ar_window = g.win;
  b.sq_b = shape->sq_b;
  b.sq_l = shape->sq_l;
  b.sq_h = shape->sq_h;
  b.sk_b = shape->sk_b;
  b.sk_l = shape->sk_l;
  b.sk_h = shape->sk_h;
  b.sv_b = shape->sv_b;
  b.sv_l = shape->sv_l;
  b.sv_h = shape->sv_h;
  b.so_b = shape->so_b;
  b.so_l = shape->so_l;
  b.so_h = shape->so_h;
  b.Q = static_cast<const uint16_t*>(Q);
  b.K = static_cast<const uint16_t*>(K);
  b.V = static_cast<const uint16_t*>(V);
  b.Qn = static_cast<const uint16_t*>(Qn ? Qn : Q);
  b.Kn = static_cast<const uint16_t*>(Kn ? Kn : K);
  b.idx = idx;
  b.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  b.sm_scale = sm_scale;
  b.Pq = static_cast<const uint16_t*>(lr->Pq);
  b.Pk = static_cast<const uint16_t*>(lr->Pk);
  b.P_hs = lr->P_head_stride;
  b.rank = lr->rank;
  b.rope_tab = w.lr.rope_tab;
  b.rope = rope_args(lr, shape);
  b.Ct_hi = w.lr.ct_hi;
  b.Ct_lo = w.lr.ct_lo;
  b.C = w.C;
  b.eps = lr->rms_eps;
  b.rmsw = static_cast<const uint16_t*>(lr->rms_weight);
  b.g = g_ptr;
  b.g_sb = g_stride_b;
  b.g_sl = g_stride_l;
  b.g_sh = g_stride_h;
  b.dO = static_cast<const uint16_t*>(dO);
  b.Os = Os;
  b.rms = rms;
  b.lse = lse;
  b.dOs = w.dOs;
  b.Dd = w.Dd;
  b.dg_head = w.dg_head;
  b.qt = w.qt;
  b.dy = w.dy;
  b.da = w.da;
  b.db = w.db;
  b.dC = w.dC;
  b.dCt_hi = w.dCt_hi;
  b.dCt_lo = w.dCt_lo;
  b.tlist = w.tlist;
  b.toff = w.toff;
  b.korder = w.korder;
  b.dQ = dQ;
  b.dK = dK;
  b.dV = dV;
  b.dQn = dQn ? dQn : w.dQn_tmp;
  b.dKn = dKn;
  b.dQn_into_dQ = dQn == nullptr;
  b.dKn_into_dK = dKn == nullptr;
  // query side: dO_s, D, dg shares, q~, dy, da, the query-side dQn
  if ((e = sd::launch_bwd_query(b, g.D, st)) != hipSuccess) return hip_fail(e, "backward, query side");
  // dC per chunk, then for each chunk the sum over the chunks that see it
  if ((e = sd::launch_token_outer(w.qt, w.dy, nullptr, 0, 0, 0, g.B, g.H, g.L, g.D, w.dC_runs, w.dC_part, st)) !=
      hipSuccess)
    return hip_fail(e, "dC sums");
  if ((e = sd::launch_dstate_finalize(w.dC_part, BH, w.dC_runs, g.n_ar, g.win, g.D, w.dC, w.dCt_hi, w.dCt_lo, st)) !=
      hipSuccess)
    return hip_fail(e, "dC finalize");
  const bool per_head = lr->P_head_stride != 0;
  if (dPq) {
    if ((e = sd::launch_token_outer(w.da, nullptr, b.Qn, shape->sq_b, shape->sq_l, shape->sq_h, g.B, g.H, g.L, g.D,
                                    w.dP_runs, w.dP_part, st)) != hipSuccess)
      return hip_fail(e, "dPq sums");
    if ((e = sd::launch_dproj_finalize(w.dP_part, g.B, g.H, w.dP_runs.n_runs, lr->rank, g.D, per_head, dPq, st)) !=
        hipSuccess)
      return hip_fail(e, "dPq finalize");
  }
  // softmax branch
  if ((e = sd::launch_transpose_map(idx, BH, g.Nq, g.Nk, k_keep, w.tlist, w.toff, w.korder, st)) != hipSuccess)
    return hip_fail(e, "map transpose");
  if ((e = sd::launch_bwd_dq(b, g.D, st)) != hipSuccess) return hip_fail(e, "backward dQ");
  if ((e = sd::launch_bwd_dkdv(b, g.D, st)) != hipSuccess) return hip_fail(e, "backward dK, dV");
  // key side of the low-rank branch (adds into dV, and into dK without Kn)
  if ((e = sd::launch_bwd_key(b, g.D, st)) != hipSuccess) return hip_fail(e, "backward, key side");
  if (dPk) {
    if ((e = sd::launch_token_outer(w.db, nullptr, b.Kn, shape->sk_b, shape->sk_l, shape->sk_h, g.B, g.H, g.L, g.D,
                                    w.dP_runs, w.dP_part, st)) != hipSuccess)
      return hip_fail(e, "dPk sums");
    if ((e = sd::launch_dproj_finalize(w.dP_part, g.B, g.H, w.dP_runs.n_runs, lr->rank, g.D, per_head, dPk, st)) !=
        hipSuccess)
      return hip_fail(e, "dPk finalize");
  }
  if (dg && (e = sd::launch_dgate(w.dg_head, g.B, g.L, g.H, g_stride_b, g_stride_l, g_stride_h, dg, st)) !=
                hipSuccess)
    return hip_fail(e, "dg");
  (void)rows;
  return ok();
}

const char* sd_status_string(int status) {
  switch (status) {
    case SD_OK: return "ok";
    case SD_ERR_INVALID_ARG: return "invalid argument";
    case SD_ERR_UNSUPPORTED: return "unsupported";
    case SD_ERR_ALIGN: return "misaligned pointer or stride";
    case SD_ERR_WORKSPACE: return "workspace too small";
    case SD_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sd_last_error(void) { return g_err.c_str(); }

}  // extern "C"
