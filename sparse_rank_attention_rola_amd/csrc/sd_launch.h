// Host-side launchers of the libsd kernels (internal; the public ABI is sd.h).
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sd_tiles.h"

namespace sd {

// Runs of 64-token tiles, each accumulating one partial low-rank state.
// Autoregressive chunk c holds tokens [c * ar_tokens, min(L, (c+1) * ar_tokens))
// (one chunk of L tokens without a causal window) and is split into
// runs_per_ar runs of at most run_tiles tiles, counted from the tile that
// holds its first token; a run counts only the tokens of its chunk, so a
// tile across a chunk boundary is read by both chunks' runs.
struct RunGeo {
  int ar_tokens;
  int runs_per_ar;
  int run_tiles;
  int n_runs;  // runs per (batch, head) = chunks * runs_per_ar
};

__host__ __device__ inline void run_extent(const RunGeo& g, int L, int run, int& t_begin, int& t_end, int& lo,
                                           int& hi) {
  const int c = run / g.runs_per_ar, j = run - c * g.runs_per_ar;
  lo = c * g.ar_tokens;
  hi = lo + g.ar_tokens < L ? lo + g.ar_tokens : L;
  const int ta = lo / 64, tb = (hi + 63) / 64;
  t_begin = ta + j * g.run_tiles < tb ? ta + j * g.run_tiles : tb;
  t_end = t_begin + g.run_tiles < tb ? t_begin + g.run_tiles : tb;
}

// Arguments of the attention-family kernels (sparse branch, low-rank query
// output, fused layer). Strides are in elements.
struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* Qn;
  int64_t sq_b, sq_l, sq_h, sk_b, sk_l, sk_h, sv_b, sv_l, sv_h, so_b, so_l, so_h;
  int B, H, L, Nq, Nk, kkeep, Hg, Wg;
  const int32_t* idx;  // [B, H, Nq, kkeep]
  float scale_log2;    // softmax scale * log2(e)
  void* out;
  int out_f32;
  float* rms;  // optional [B, L, H]
  float* lse;  // optional [B, H, L] (head-major), sparse mode: m + log2(l) of the scaled scores
  // fused mode, optional: O_s (bf16 [B, L, H, D] contiguous) with rms and lse
  // as above, kept for the backward
  uint16_t* os_save;
  // low-rank branch
  const uint16_t* Pq;
  int64_t P_hs;
  int rank;
  const float2* rope_tab;  // [n pairs][max_ext] (cos, sin)
  RopeArgs rope;
  const uint16_t* Ct_hi;  // bf16 [B*H, D, 32], state C transposed, hi part
  const uint16_t* Ct_lo;  // lo part
  float eps;
  const uint16_t* rmsw;  // optional bf16 [D]
  // gate
  const float* g;
  int64_t g_sb, g_sl, g_sh;
  // causal window: query i sees the keys of autoregressive chunks
  // i/ar_tokens - ar_window + 1 .. i/ar_tokens (ar_window 0: all earlier
  // chunks); ar_tokens = L and ar_window = 0 without one. The state of the
  // chunk is Ct_*[(b*H + h) * n_ar + chunk].
  int ar_tokens, ar_window;
};

struct LowrankKvArgs {
  const uint16_t* Kn;
  const uint16_t* V;
  int64_t sk_b, sk_l, sk_h, sv_b, sv_l, sv_h;
  int B, H, L, Hg, Wg;
  RunGeo runs;
  const uint16_t* Pk;
  int64_t P_hs;
  int rank;
  const float2* rope_tab;
  RopeArgs rope;
  float* partial;  // [B*H, runs.n_runs, 32, D]
};

// One streaming pass over Kn, V: block means of K (when Kn is K and kmean is
// set) plus the partial low-rank states of each run of tiles.
struct PrepareArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* Kn;  // may equal K
  const uint16_t* V;
  int64_t sq_b, sq_l, sq_h, sk_b, sk_l, sk_h, sv_b, sv_l, sv_h;
  int B, H, L, Nq, Nk, block_q, Hg, Wg;
  float rcp_hw, rcp_wg;  // 1 / (Hg * Wg) and 1 / Wg rounded to float
  RunGeo runs;  // without a causal window, run_tiles is a multiple of block_q / 64
  const uint16_t* Pk;
  int64_t P_hs;
  int rank;
  const float2* rope_tab;
  RopeArgs rope;
  // rank slots of the stream pass: slot i holds rank slot_rank[i] (-1:
  // empty); slots 2p, 2p+1 form RoPE pair slot_pair[p] (-1: not rotated)
  int8_t slot_rank[32];
  int8_t slot_pair[16];
  uint32_t slot_mask;  // bit i set where slot_rank[i] >= 0
  double* kmean;   // [B*H, Nk, D] or null
  float* partial;  // [B*H, runs.n_runs, 32, D]
};

// Fused q/k RMSNorm + backbone 3D RoPE.
constexpr int kQkMaxPairs = 64;  // pairs per head (d <= 128)
struct QkNormRopeArgs {
  const uint16_t* q;  // [B*L rows][H*d], row stride ld_in elements
  const uint16_t* k;
  int64_t ld_in;
  const uint16_t* gamma_q;  // bf16 [H*d] or null (ones)
  const uint16_t* gamma_k;
  float eps;
  int B, L, H, d, Hg, Wg;
  // per pair index m = dim / 2 of a head: axis of the pair starting at
  // dim 2m (-1: the channels are not rotated) and its frequency
  int8_t pair_axis[kQkMaxPairs];
  float pair_theta[kQkMaxPairs];
  uint16_t* Q;  // outputs, bf16 [B, L, H, d] contiguous
  uint16_t* K;
  uint16_t* Qn;
  uint16_t* Kn;
  // optional block means of Q and K (f64 [B, H, ceil(L / block), d]); rows
  // go in segments of seg_rows (<= 128), a multiple of both block sizes
  double* qmean;
  double* kmean;
  int block_q, block_k, seg_rows;
  double rcp_block_q, rcp_block_k;  // 1 / block (exact: powers of two)
};
hipError_t launch_qk_norm_rope(const QkNormRopeArgs& a, hipStream_t stream);

// W8A8 FP8 projection y = diag(sx) (xq wq^T) diag(sw), bf16 out.
struct GemmFp8Args {
  const uint8_t* xq;  // [M, K], row stride ldx bytes
  const uint8_t* wq;  // [N, K], row stride ldw bytes
  const float* sx;    // [M]
  const float* sw;    // [N]
  uint16_t* y;        // [M, N] bf16, row stride ldy elements
  int64_t M, N, K, ldx, ldw, ldy;
};
hipError_t launch_gemm_fp8(const GemmFp8Args& a, hipStream_t stream);

hipError_t launch_quant_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                            float* scales, hipStream_t stream);
hipError_t launch_quant_fp8_gate(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                                 float* scales, const uint16_t* wgate, float gate_bias, float* g, hipStream_t stream);
hipError_t launch_pool_blocks(const uint16_t* X, int64_t sb, int64_t sl, int64_t sh, int B, int L, int H, int D,
                              int bs, double* out, hipStream_t stream);
// Which key blocks a row of the block map may keep, and where it goes.
// Row r of the map belongs to query block r % Nq; it is computed from row
// r % s_rows of S and written to every one of n_rep copies of the map
// (rep_stride int32 apart). Key block c is allowed for query block b when
// some query of b sees some key of c under the causal window (AttnArgs).
struct MapRule {
  int Nq, bq, bk, L;
  int ar_tokens, ar_window;
  int64_t s_rows;
  int n_rep;
  int64_t rep_stride;
};
hipError_t launch_select_topk(const double* qmean, const double* kmean, int BH, int Nk, int D, int k,
                              const MapRule& rule, uint16_t* khi, uint16_t* klo, double* knorm2, int32_t* idx,
                              hipStream_t stream);
hipError_t launch_topk_rows(const double* S, int64_t n_rows, int C, int k, const MapRule& rule, int32_t* idx,
                            hipStream_t stream);
// Fixed spatio-temporal scores: S[b][c] = -|centroid_q(b) - centroid_k(c)|^2
// in latent (t, h, w) units; cq / ck: scratch of 3 * Nq / 3 * Nk doubles.
hipError_t launch_fixed_scores(int L, int Nq, int Nk, int bq, int bk, int Hg, int Wg, double* cq, double* ck,
                               double* S, hipStream_t stream);
hipError_t launch_sparse_attn(const AttnArgs& a, int D, int BQ, hipStream_t stream);
hipError_t launch_lowrank_query(const AttnArgs& a, int D, int BQ, hipStream_t stream);
hipError_t launch_rola_fused(const AttnArgs& a, int D, int BQ, hipStream_t stream);
struct RopeThetas {
  float theta[kMaxRopePairs];
};
hipError_t launch_rope_table(const RopeThetas& th, int n, int max_ext, float2* tab, hipStream_t stream);
hipError_t launch_lowrank_kv(const LowrankKvArgs& a, int D, hipStream_t stream);
// Row of the partial states that holds each rank (-1: none, the rank's
// state is zero).
struct RankRows {
  int8_t row[32];
};
// C of autoregressive chunk c = the sum, in run order, of the partial states
// of chunks max(0, c - window + 1) .. c (window 0: 0 .. c); outputs per
// (batch, head, chunk): C_out [rank][D] f32 (optional), Ct_hi/lo [D][32].
hipError_t launch_lowrank_finalize(const float* partial, int BH, const RunGeo& runs, int n_ar, int window, int rank,
                                   int D, const RankRows& rows, float* C_out, uint16_t* Ct_hi, uint16_t* Ct_lo,
                                   hipStream_t stream);
hipError_t launch_prepare_stream(const PrepareArgs& a, int D, hipStream_t stream);

// Backward of the fused layer (block map fixed). Per-token buffers are
// contiguous [B, L, H, ...]; Q/Qn share the sq_* strides, K/Kn the sk_*, V
// the sv_* and dO the so_*.
struct BwdArgs {
  int B, H, L, Nq, Nk, kkeep, Hg, Wg, block_q;
  int ar_tokens, ar_window;
  int64_t sq_b, sq_l, sq_h, sk_b, sk_l, sk_h, sv_b, sv_l, sv_h, so_b, so_l, so_h;
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* Qn;  // may equal Q
  const uint16_t* Kn;  // may equal K
  const int32_t* idx;  // [B, H, Nq, kkeep]
  float scale_log2, sm_scale;
  // low-rank branch
  const uint16_t* Pq;
  const uint16_t* Pk;
  int64_t P_hs;
  int rank;
  const float2* rope_tab;
  RopeArgs rope;
  const uint16_t* Ct_hi;  // [B*H, n_ar, D, 32] state transposed, hi / lo
  const uint16_t* Ct_lo;
  const float* C;  // [B*H, n_ar, rank, D] state rows
  float eps;
  const uint16_t* rmsw;
  const float* g;
  int64_t g_sb, g_sl, g_sh;
  const uint16_t* dO;  // bf16 at so_*
  // forward intermediates
  const uint16_t* Os;  // bf16 [B, L, H, D] contiguous
  const float* rms;  // [B, L, H]
  const float* lse;  // [B, H, L] (head-major)
  // backward intermediates
  uint16_t* dOs;   // bf16 [B, L, H, D]
  float* Dd;       // [B, H, L] (head-major): dO_s . O_s
  float* dg_head;  // [B, L, H]
  float* qt;       // [B, L, H, 32] q~
  float* dy;       // [B, L, H, D]
  float* da;       // [B, L, H, 32]
  float* db;       // [B, L, H, 32]
  const float* dC;        // [B*H, n_ar, 32, D]: for chunk c, the sum of dC over the chunks that see c
  const uint16_t* dCt_hi;  // [B*H, n_ar, D, 32] the same transposed, hi / lo
  const uint16_t* dCt_lo;
  // key-block -> query-block lists
  const int32_t* tlist;  // [B*H, Nq*kkeep]
  const int32_t* toff;   // [B*H, Nk + 1]
  const int32_t* korder; // [B*H, Nk]: each head's key blocks, the most kept first
  // outputs, f32 [B, L, H, D]
  float* dQ;
  float* dK;
  float* dV;
  float* dQn;  // receives the low-rank query-side gradient (may be a workspace buffer)
  float* dKn;
  int dQn_into_dQ, dKn_into_dK;  // the branch read Q / K: add into dQ / dK
};
hipError_t launch_bwd_query(const BwdArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_key(const BwdArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int D, hipStream_t stream);
hipError_t launch_transpose_map(const int32_t* idx, int BH, int Nq, int Nk, int k, int32_t* tlist, int32_t* toff,
                                int32_t* korder,
                                hipStream_t stream);
// Partial sums over runs of tokens of X^T Y, X [rows][32] f32 (contiguous,
// row = token*H + head), Y [rows][D] (f32 contiguous when Yf, else bf16 at
// token stride y_sl and head stride y_sh): part[(bh * runs.n_runs + run)][32][D].
hipError_t launch_token_outer(const float* X, const float* Yf, const uint16_t* Yb, int64_t y_sb, int64_t y_sl,
                              int64_t y_sh, int B, int H, int L, int D, const RunGeo& runs, float* part,
                              hipStream_t stream);
// Gradient of the state seen by each chunk: for (bh, chunk c) the sum of the
// run partials of chunks c .. c + window - 1 (window 0: c .. last), written
// as rows f32 [32][D] and transposed bf16 hi / lo [D][32].
hipError_t launch_dstate_finalize(const float* part, int BH, const RunGeo& runs, int n_ar, int window, int D,
                                  float* dC, uint16_t* dCt_hi, uint16_t* dCt_lo, hipStream_t stream);
// dP [n_out][rank][D] = the sum of the run partials of every (b, h) (n_out = 1)
// or of every b for each h (n_out = H), in a fixed order.
hipError_t launch_dproj_finalize(const float* part, int B, int H, int n_runs, int rank, int D, bool per_head,
                                 float* dP, hipStream_t stream);
// dg from the per-(token, head) shares: summed over the heads when g_sh == 0.
hipError_t launch_dgate(const float* dg_head, int B, int L, int H, int64_t g_sb, int64_t g_sl, int64_t g_sh,
                        float* dg, hipStream_t stream);
hipError_t launch_gate_fuse(const void* Os, const void* Olr, int in_f32, const float* g, int64_t g_sb, int64_t g_sl,
                            int64_t g_sh, void* O, int B, int L, int H, int D, int64_t so_b, int64_t so_l,
                            int64_t so_h, hipStream_t stream);

}  // namespace sd
