/*
 * sd.h -- C ABI of libsd: RoLA compensated sparse attention and per-token
 * FP8 E4M3 activation quantisation on AMD Instinct MI355X (gfx950).
 *
 * The method (robotworld.top SparkDiffusion write-up, section 2.1,
 * "compensated sparse attention"): the attention of a video DiT is replaced
 * by a block-sparse softmax branch A_M that keeps a 1-s fraction of the
 * query/key blocks plus a low-rank compensation branch, fused per token:
 *     q~_i = R_r(p_i) phi(P_q qn_i),  k~_j = R_r(p_j) phi(P_k kn_j),
 *     C = sum_j k~_j v_j^T,           O_lr,i = RMSNorm(q~_i^T C),
 *     O_i = O_s,i + g_i r_i O_lr,i    (r_i = RMS of the sparse output O_s,i).
 * The FP8 quantiser is the deployment step of section 2.3 of the same page.
 *
 * Conventions shared by every entry point:
 *  - Device pointers are HIP device memory owned by the caller. The library
 *    never allocates or frees; scratch space is a caller-provided workspace
 *    whose size the matching *_workspace_size function returns.
 *  - Per-token tensors are bf16 (or f32 where stated) in [B, L, H, d]
 *    layout: the d elements of one (batch, token, head) are contiguous and
 *    the three outer strides are given in ELEMENTS (int64). Strides and the
 *    base pointers must keep every 8-element (16-byte) group aligned.
 *  - Tokens are in raster order of a T x Hg x Wg latent grid:
 *    token i sits at p_i = (t, h, w) with i = (t*Hg + h)*Wg + w.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call is
 *    asynchronous and stream-ordered; nothing synchronises the host. The
 *    prepare phase (sd_rola_prepare, sd_rola_attention) may run part of its
 *    work on a second stream the library creates once per device and keeps
 *    until the process ends; events fork it from `stream` and join it back,
 *    so the call stays ordered on `stream`, also when a launch fails. A call
 *    on a stream that is being captured into a graph runs all of its work
 *    on that stream: the second stream is shared by every host thread, and
 *    forking it into one thread's capture would record another thread's
 *    eager work into that graph.
 *  - Return value: SD_OK (0) or an SD_ERR_* code. Arguments are validated
 *    on the host before anything is launched; on a validation error no
 *    device memory is touched. sd_last_error() gives a thread-local message.
 *    SD_ERR_HIP reports a launch failure seen right after launching.
 *  - Calls are thread-safe: the library keeps no state beyond the
 *    thread-local error text and that second stream, whose use a mutex
 *    serialises.
 */
#ifndef SD_H_
#define SD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sd_status {
  SD_OK = 0,
  SD_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shape   */
  SD_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels do   */
  SD_ERR_ALIGN = 3,       /* pointer or stride breaks 16-byte alignment  */
  SD_ERR_WORKSPACE = 4,   /* workspace missing or too small              */
  SD_ERR_HIP = 5          /* the HIP runtime reported an error           */
};

enum sd_dtype { SD_DTYPE_BF16 = 1, SD_DTYPE_F32 = 2 };

enum sd_phi { SD_PHI_ELU1 = 1 }; /* phi(x) = ELU(x) + 1 */

/* Selector of the sparse branch (robotworld.top write-up, section 2.1: the
 * kept 1-s of the blocks come from top-k over block-level scores or from a
 * fixed spatio-temporal pattern). */
enum sd_select {
  SD_SELECT_TOPK = 0,  /* top-k of mean(Q block) . mean(K block)            */
  SD_SELECT_FIXED = 1  /* the k key blocks whose centroids in latent
                          (t, h, w) units are nearest the query block's
                          (squared distance -((dt^2 + dh^2) + dw^2), float64
                          without fused multiply-add; needs the grid)       */
};

/* Geometry of one attention layer. Supported: d in {64, 128},
 * block_q in {64, 128}, block_k == 64, L <= 131072, B, H >= 1.
 * T, Hg, Wg are needed (T*Hg*Wg == L) only by the low-rank branch, the fused
 * entry and SD_SELECT_FIXED; the scored block map and the sparse branch
 * ignore them.
 * s?_b, s?_l, s?_h: element strides of Q, K, V and of every output tensor
 * (so_*) in [B, L, H, d] layout.
 * select: SD_SELECT_TOPK or SD_SELECT_FIXED (used by the block map).
 * chunk_tokens, window: causal window for autoregressive generation
 * (robotworld.top write-up, section 4: compensated sparse attention
 * restricted to a causal window). chunk_tokens = 0: bidirectional (window
 * must be 0). Otherwise tokens form chunks of chunk_tokens consecutive
 * tokens (a chunk of f latent frames is f*Hg*Wg tokens; at most 4096
 * chunks) and a query of chunk c sees exactly the keys of chunks
 * c-window+1 .. c (window 0: 0 .. c), in both branches: the block map keeps
 * only key blocks some query of the block sees (rows with fewer than k_keep
 * such blocks keep them all and are padded with -1), the sparse branch
 * masks the other keys of a kept block (a query that sees none of the kept
 * keys gets O_s = 0), and the low-rank state of a chunk sums k~ v^T over
 * the keys its queries see. Zero-initialised fields give the bidirectional
 * scored layer. */
typedef struct sd_attn_shape {
  int32_t B, H, L, d;
  int32_t T, Hg, Wg;
  int32_t block_q, block_k;
  int64_t sq_b, sq_l, sq_h;
  int64_t sk_b, sk_l, sk_h;
  int64_t sv_b, sv_l, sv_h;
  int64_t so_b, so_l, so_h;
  int32_t select;
  int32_t chunk_tokens;
  int32_t window;
} sd_attn_shape;

/* One rotated pair of the rank-truncated 3D RoPE R_r(p): feature dims
 * (dim, dim+1) rotate by the angle p_axis * theta, axis 0/1/2 = t/h/w. */
typedef struct sd_rope_pair {
  int32_t dim;
  int32_t axis;
  float theta;
} sd_rope_pair;

/* Parameters of the low-rank branch (robotworld.top write-up, section 2.1,
 * q~/k~ and O_lr equations; kais-engine report, section 2.1: proj_q and
 * proj_k map head_dim to rank).
 *  rank        16 or 32.
 *  phi         SD_PHI_ELU1.
 *  Pq, Pk      device bf16 [rank, d] row-major projections; head h uses
 *              P + h * P_head_stride (0 = one matrix shared by all heads).
 *  rope        HOST array of n_rope pairs (read during the call only); the
 *              pairs must not overlap; dims not in any pair are not rotated.
 *  rms_eps     epsilon of the RMSNorm of O_lr.
 *  rms_weight  device bf16 [d] RMSNorm weight, 8-byte aligned (else
 *              SD_ERR_ALIGN), or NULL for ones. */
typedef struct sd_lowrank_params {
  int32_t rank;
  int32_t phi;
  const void* Pq;
  const void* Pk;
  int64_t P_head_stride;
  const sd_rope_pair* rope;
  int32_t n_rope;
  float rms_eps;
  const void* rms_weight;
} sd_lowrank_params;

/* Key blocks kept per query block at sparsity s: ceil((1-s)*n_kblocks)
 * clamped to [1, n_kblocks] (SparkDiffusion README_zh, single-sample
 * inference: `topk` is the kept fraction, 0.1/0.05/0.03 = 90/95/97%).
 * Returns -1 if n_kblocks < 1 or s is outside [0, 1). Host only. */
int sd_keep_count(double sparsity, int n_kblocks);

/* Fills out[0..max_pairs) with the default rank-truncated 3D RoPE: the
 * rank dims split over (t, h, w) as (r - 2*floor(r/3), floor(r/3),
 * floor(r/3)), adjacent pairs inside each axis block, theta_m =
 * base^(-2m/n_axis), an odd last dim of a block left unrotated. Returns the
 * number of pairs, or -1 on bad arguments. Host only. */
int sd_rope_default(int rank, double base, sd_rope_pair* out, int max_pairs);

/* ---- (1) block map --------------------------------------------------------
 * robotworld.top write-up, section 2.1: the sparse branch keeps the top-k
 * key blocks per query block by a block-level score. Score of query block b
 * and key block c = mean(Q over b) . mean(K over c), means over the valid
 * tokens of (possibly partial) blocks, accumulated and compared in float64.
 * idx: device int32 [B, H, Nq, k_keep], Nq = ceil(L/block_q); each row lists
 * the k_keep highest-scoring key blocks (equal scores: lower index first)
 * in ascending order. 1 <= k_keep <= Nk = ceil(L/block_k).
 * shape->select = SD_SELECT_FIXED scores by the fixed spatio-temporal
 * pattern instead (Q and K are not read; every (b, h) gets the same map).
 * Under a causal window only allowed blocks are candidates and short rows
 * end in -1 (see sd_attn_shape). */
size_t sd_block_select_workspace_size(const sd_attn_shape* shape);
int sd_block_select(const sd_attn_shape* shape, const void* Q, const void* K, int k_keep,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* ---- (2) sparse softmax branch A_M --------------------------------------
 * robotworld.top write-up, section 2.1 (A_M over the kept 1-s of the
 * blocks; the dense-attention equation for the softmax form). Every query
 * of query block qb of (batch b, head h) attends with softmax(q.k * sm_scale)
 * to the valid keys of the blocks idx[b, h, qb, :] (bf16 operands, f32
 * accumulation). Entries outside [0, Nk) select no keys.
 * Os: [B, L, H, d] at the so_* strides, bf16 or f32 (os_dtype).
 * rms: optional device f32 [B, L, H] (contiguous) = RMS over d of each
 * O_s row (the r_i of the fusion), or NULL. */
int sd_sparse_attn(const sd_attn_shape* shape, const void* Q, const void* K, const void* V,
                   const int32_t* idx, int k_keep, float sm_scale, void* Os, int os_dtype,
                   float* rms, void* stream);

/* ---- (3) low-rank branch ---------------------------------------------------
 * robotworld.top write-up, section 2.1, the q~/k~ and C/O_lr equations:
 * C[b,h] = sum over all L tokens of k~_j v_j^T (f32 [rank, d]), then
 * O_lr,i = w * y / sqrt(mean(y^2) + eps) with y = q~_i^T C. Under a causal
 * window every chunk c has its own C (the keys its queries see).
 * Qn, Kn: the normalised q/k the branch reads (strides of Q and K).
 * Olr: [B, L, H, d] at the so_* strides, bf16 or f32 (olr_dtype).
 * C_out: optional device f32 [B, H, n_chunks, rank, d] (n_chunks =
 * ceil(L / chunk_tokens), 1 without a causal window), or NULL. */
size_t sd_lowrank_workspace_size(const sd_attn_shape* shape, const sd_lowrank_params* lr);
int sd_lowrank_attn(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Qn,
                    const void* Kn, const void* V, void* Olr, int olr_dtype, float* C_out,
                    void* ws, size_t ws_bytes, void* stream);

/* ---- (4) gated fusion ------------------------------------------------------
 * robotworld.top write-up, section 2.1, the O_i equation:
 * O = O_s + g * r * O_lr with r the RMS over d of the O_s row (computed
 * here from Os). Os, Olr: in_dtype at the so_* strides; O: bf16 at the
 * so_* strides (may alias neither input). g: device f32, the gate of
 * (b, token, head) at g[b*g_stride_b + i*g_stride_l + h*g_stride_h]
 * (g_stride_h = 0: one gate per token). */
int sd_gate_fuse(const sd_attn_shape* shape, const void* Os, const void* Olr, int in_dtype,
                 const float* g, int64_t g_stride_b, int64_t g_stride_l, int64_t g_stride_h,
                 void* O, void* stream);

/* ---- (5) per-token FP8 E4M3 quantisation ---------------------------------
 * robotworld.top write-up, section 2.3: a dynamic scale per token (row),
 * scale and conversion in one pass over memory. For row m of x (bf16,
 * M x K, row stride ldx elements):
 *   amax = max(max_k |x_mk|, 1e-12f),  scales[m] = amax / 448 (f32),
 *   q_mk = E4M3FN(fl32(x_mk * fl32(448 / amax))), nearest-even, saturating.
 * scales are the dequantisation multipliers. q: uint8 codes, row stride ldq.
 * Needs K % 8 == 0, ldx % 8 == 0, ldq % 8 == 0, K <= 16384, x 16-byte and
 * q 8-byte aligned. Non-finite inputs give unspecified codes. M = 0 (no
 * rows) does nothing and returns SD_OK; the pointers may then be NULL. */
int sd_quant_fp8_per_token(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                           int64_t ldq, float* scales, void* stream);

/* The same quantiser with the block's scalar gate computed from the same
 * row in the same pass (kais-engine report, section 2.1: the gate is
 * gate_proj(x) + gate_bias, one scalar per token; robotworld.top write-up,
 * section 2.1: O_i = O_s,i + g_i r_i O_lr,i):
 *   g[m] = b_gate + sum_k w_gate[k] * x_mk      (f32 accumulation)
 * w_gate: bf16 [K], 16-byte aligned; g: f32 [M]. Codes and scales as in
 * sd_quant_fp8_per_token (bit-identical), same requirements. */
int sd_quant_fp8_gate(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                      const void* w_gate, float b_gate, float* g, void* stream);

/* ---- (6) W8A8 FP8 projection ------------------------------------------------
 * robotworld.top write-up, section 2.3: the linear projections run W8A8 in
 * FP8 E4M3, weights with a static scale per output channel, activations with
 * the dynamic per-token scale of sd_quant_fp8_per_token:
 *   y[m, n] = sx[m] * sw[n] * sum_k E4M3(xq[m, k]) * E4M3(wq[n, k])
 * xq: uint8 codes [M, K], row stride ldx bytes (the quantiser's q);
 * sx: f32 [M] (its scales); wq: uint8 codes [N, K], row stride ldw bytes,
 * one row per output channel (W quantised row by row, e.g. by
 * sd_quant_fp8_per_token on W once, offline); sw: f32 [N]; y: bf16 [M, N],
 * row stride ldy elements, rounded to nearest even. Accumulation is f32.
 * Needs K % 64 == 0, ldx and ldw multiples of 16 (>= K), ldy % 4 == 0
 * (>= N), 16-byte aligned xq, wq, sw and 8-byte aligned y; K <= 65536 and
 * 256 * max(ldx, ldw) < 2^31. All buffers are caller-owned device memory. */
int sd_gemm_fp8_w8a8(const uint8_t* xq, int64_t M, int64_t K, int64_t ldx, const float* sx,
                     const uint8_t* wq, int64_t N, int64_t ldw, const float* sw, void* y, int64_t ldy,
                     void* stream);

/* ---- (7) q/k producer of the attention block --------------------------------
 * robotworld.top write-up, section 2.1: the low-rank branch reuses the
 * normalised q/k from before the backbone attention, which applies its own
 * 3D RoPE; kais-engine report, section 2.1: fused QKV + RoPE operator.
 * For every token row x (H*d channels) of q and of k (bf16, rows of B*L
 * tokens in (b, l) order, row stride ld_in elements, e.g. slices of the
 * W8A8 QKV projection's output):
 *   y_c = x_c / sqrt(mean_c' x_c'^2 + eps) * gamma_c      -> Qn, Kn (bf16)
 *   per head: pairs (dim, dim+1) of y rotated by p_axis * theta -> Q, K
 * with p = (t, h, w) of token l = (t*Hg + h)*Wg + w. Computation in f32,
 * each output rounded once to bf16 (nearest even). Outputs are contiguous
 * [B, L, H, d]. gamma_q / gamma_k: bf16 [H*d], or NULL for ones. rope: host
 * array of n_rope pairs (e.g. sd_rope_default(d, 10000, ...)); channels in
 * no pair are copied unrotated.
 * Optionally (qmean / kmean non-NULL) it also writes the block means of the
 * rotated Q and K, the q-bar / k-bar of the block scores (section 2.1):
 * float64 [B, H, ceil(L / block), d], each the exact float64 sum of the
 * block's stored bf16 values in token order divided by its token count
 * (the tail block by its own count); block_q in {64, 128}, block_k = 64.
 * sd_rola_prepare takes them instead of pooling Q and K itself.
 * Needs d in {64, 128}, H*d <= 8192, T*Hg*Wg == L, every pair's dim even
 * (pairs inside 8-channel groups), ld_in >= H*d and a multiple of 8, all
 * bf16 device buffers 16-byte aligned, the means 8-byte aligned. Errors
 * leave the outputs unwritten. */
int sd_qk_norm_rope(int B, int L, int H, int d, int T, int Hg, int Wg, const void* q, const void* k,
                    int64_t ld_in, const void* gamma_q, const void* gamma_k, float eps, const sd_rope_pair* rope,
                    int n_rope, void* Q, void* K, void* Qn, void* Kn, double* qmean, double* kmean, int block_q,
                    int block_k, void* stream);

/* ---- fused layer -------------------------------------------------------------
 * The whole path of section 2.1 in one call: block map, sparse branch,
 * low-rank branch and gated fusion. O: bf16 [B, L, H, d] at the so_*
 * strides. Qn/Kn may be NULL to read Q/K. g as in sd_gate_fuse. idx_out:
 * optional device int32 [B, H, Nq, k_keep] receiving the block map used
 * (NULL keeps it in the workspace). */
size_t sd_rola_workspace_size(const sd_attn_shape* shape, const sd_lowrank_params* lr, int k_keep);
int sd_rola_attention(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q,
                      const void* K, const void* V, const void* Qn, const void* Kn, const float* g,
                      int64_t g_stride_b, int64_t g_stride_l, int64_t g_stride_h, int k_keep,
                      float sm_scale, void* O, int32_t* idx_out, void* ws, size_t ws_bytes,
                      void* stream);

/* The fused layer in two phases, for callers that schedule or time them
 * apart (sd_rola_attention is exactly prepare followed by apply):
 *  sd_rola_prepare  block map (into idx_out, or the workspace when NULL) and
 *                   the low-rank state C (into the workspace);
 *  sd_rola_apply    the fused sparse + low-rank + gate kernel; it reads the
 *                   block map from idx (NULL: the workspace) and C from the
 *                   workspace left by sd_rola_prepare with the same shape,
 *                   parameters, k_keep and workspace, earlier on the stream.
 * Arguments mean what they mean for sd_rola_attention. qmean / kmean: NULL
 * (prepare pools Q and K itself) or both the float64 block means of Q and K,
 * [B, H, Nq, d] and [B, H, Nk, d] contiguous, as sd_qk_norm_rope writes them
 * (read by the scored selector only; the caller keeps them until the call's
 * work on the stream is done). */
int sd_rola_prepare(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                    const void* V, const void* Qn, const void* Kn, const double* qmean, const double* kmean,
                    int k_keep, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);
int sd_rola_apply(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                  const void* V, const void* Qn, const float* g, int64_t g_stride_b, int64_t g_stride_l,
                  int64_t g_stride_h, int k_keep, float sm_scale, void* O, const int32_t* idx, void* ws,
                  size_t ws_bytes, void* stream);

/* The forward quantities the backward needs, kept by the forward of a
 * training step (sd_rola_apply_save) so that the backward does not form them
 * again. All device memory owned by the caller:
 *   Os:  bf16 [B, L, H, d] contiguous, the sparse branch output O_s (before
 *        the gated fusion);
 *   rms: f32 [B, L, H] contiguous, the RMS over d of each O_s row (r_i);
 *   lse: f32 [B, H, L] contiguous (head-major), the log2-domain log-sum-exp
 *        of each query's scaled scores over its kept keys, +inf where the
 *        query saw no key. */
typedef struct sd_rola_saved {
  void* Os;
  float* rms;
  float* lse;
} sd_rola_saved;

/* For callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid allocation): sd_rola_attention without a
 * workspace. Its scratch is a static device array of SD_NOALLOC_SCRATCH_BYTES
 * (128 MiB: enough for the Wan2.1-14B 720P layer at 90% and 97% sparsity),
 * held by every GPU the library runs on until the process ends. Shapes whose
 * sd_rola_workspace_size exceeds it return SD_ERR_UNSUPPORTED. Nothing is
 * allocated or freed, and no second stream is used: all work is ordered on
 * `stream`. Every call on one GPU shares that GPU's array (nothing in it has
 * to start at zero: each call writes what it reads), so calls that overlap on
 * one GPU, from other streams or threads, race. Other arguments as for
 * sd_rola_attention; idx_out may be NULL. */
#define SD_NOALLOC_SCRATCH_BYTES (128u << 20)
int sd_rola_attention_noalloc(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q,
                              const void* K, const void* V, const void* Qn, const void* Kn, const float* g,
                              int64_t g_stride_b, int64_t g_stride_l, int64_t g_stride_h, int k_keep,
                              float sm_scale, void* O, int32_t* idx_out, void* stream);

/* sd_rola_apply that also writes the quantities of an sd_rola_saved, the same
 * values the backward would form itself, bit for bit. */
int sd_rola_apply_save(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                       const void* V, const void* Qn, const float* g, int64_t g_stride_b, int64_t g_stride_l,
                       int64_t g_stride_h, int k_keep, float sm_scale, void* O, const int32_t* idx, void* ws,
                       size_t ws_bytes, const sd_rola_saved* save, void* stream);

/* ---- (8) backward of the fused layer -----------------------------------------
 * SparkDiffusion README_zh, distillation and operators sections: training
 * the sparse student needs a backward kernel of its sparse + low-rank
 * attention. The gradients are the exact derivatives of the forward of
 * sd_rola_attention (robotworld.top write-up, section 2.1, under the causal
 * window of the shape when it has one) with the block map `idx` held fixed
 * (the map the forward used, e.g. idx_out of sd_rola_prepare):
 *   dO: bf16 [B, L, H, d] at the so_* strides, the gradient of O.
 *   dQ, dK, dV: f32 [B, L, H, d] contiguous (required, fully written).
 *   dQn, dKn: f32 [B, L, H, d] contiguous, the gradient reaching the
 *     low-rank branch's separate inputs; give them exactly when Qn / Kn are
 *     given. With Qn (Kn) NULL the branch reads Q (K) and its gradient is
 *     added into dQ (dK).
 *   dPq, dPk: f32 [rank, d] (P_head_stride 0) or [H, rank, d], or NULL to
 *     skip them.
 *   dg: f32 at the gate's strides, or NULL to skip it. A stride of 0 is a
 *     broadcast and dg sums over that dimension (g_stride_h 0: over the
 *     heads; g_stride_b 0: over the batch; g_stride_l 0: over the tokens), in
 *     a fixed order. The non-zero strides must not overlap (SD_ERR_UNSUPPORTED
 *     otherwise: elements of dg would be written by several (b, l, h)).
 *   saved: the forward's O_s, RMS and log-sum-exp (sd_rola_apply_save with
 *     the same inputs and block map), or NULL to form them here.
 * The low-rank state is formed again inside. All sums run in a fixed order
 * (the result is bitwise reproducible, and the same with or without saved).
 * Needs (L + 64) * max(H * d, sq_l) * 2 < 2^32. */
size_t sd_rola_backward_workspace_size(const sd_attn_shape* shape, const sd_lowrank_params* lr, int k_keep);
int sd_rola_backward(const sd_attn_shape* shape, const sd_lowrank_params* lr, const void* Q, const void* K,
                     const void* V, const void* Qn, const void* Kn, const float* g, int64_t g_stride_b,
                     int64_t g_stride_l, int64_t g_stride_h, int k_keep, float sm_scale, const int32_t* idx,
                     const sd_rola_saved* saved, const void* dO, float* dQ, float* dK, float* dV, float* dQn,
                     float* dKn, float* dPq, float* dPk, float* dg, void* ws, size_t ws_bytes, void* stream);

const char* sd_status_string(int status);
const char* sd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SD_H_ */
