// Block map of the sparse branch: mean pooling, block scores, exact top-k.
//
// robotworld.top SparkDiffusion write-up, section 2.1: the sparse branch A_M
// keeps a 1-s fraction of the query/key blocks, chosen by top-k over a
// block-level score. Here the score of query block b and key block c is the
// dot product of the block means of Q and K.
//
// The score decides an integer (which blocks are kept), so it is formed in
// float64: the block sums of <= 128 bf16 values are exact in float64, the
// means are IEEE divisions, and only the summation order of the 64/128-term
// dot product can differ from a plain float64 evaluation.
//
//  pool_blocks_kernel  Q or K [B, L, H, d] bf16 -> means [B, H, n_blocks, d] f64.
//                      Each thread owns 8 adjacent channels of one head and
//                      walks the tokens of one block; a wave reads 1 KB of a
//                      token row per load (coalesced), HBM-bound.
//  kmean_split_kernel,  the scored selector: approximate scores of a row
//  select_topk_kernel  on MFMA, then exact float64 scores only for the few
//                      key blocks near its k-th score, and the exact top-k
//                      (described where they are defined).
//  fixed_scores_kernel the fixed spatio-temporal pattern (same section: a
//                      fixed pattern may replace the scored selection):
//                      minus the squared distance of the block centroids in
//                      latent (t, h, w) coordinates.
//  topk_rows_kernel    one wavefront per row of fixed-pattern scores: a
//                      radix select on 8-bit digits of the order-preserving
//                      64-bit image of the scores, from the top, finds the
//                      k-th largest score
//                      exactly (it stops early once every candidate left in
//                      the chosen bin is kept); the row is then compacted in
//                      index order with ballots, so the output is ascending
//                      and equal scores at the threshold go to the lower
//                      block index. Under a causal window (section 4 of the
//                      write-up, autoregressive extension) only the key
//                      blocks some query of the row's block may see are
//                      candidates; a row with fewer than k of them keeps
//                      them all and is padded with -1.
#include "sd_device.h"
#include "sd_launch.h"

namespace sd {

__global__ __launch_bounds__(256) void pool_blocks_kernel(const uint16_t* __restrict__ X, int64_t sb, int64_t sl,
                                                          int64_t sh, int L, int H, int D, int bs, int nblk,
                                                          double* __restrict__ out) {
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  const int cpr = D >> 3;  // 8-channel chunks per head
  const int chunk = blockIdx.z * 256 + threadIdx.x;
  if (chunk >= H * cpr) return;
  const int h = chunk / cpr;
  const int d0 = (chunk - h * cpr) * 8;
  const int t0 = blk * bs;
  const int t1 = min(L, t0 + bs);
  const uint16_t* p = X + (int64_t)b * sb + (int64_t)h * sh + d0;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  int t = t0;
  for (; t + 4 <= t1; t += 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const u32x4*>(p + (int64_t)(t + u) * sl);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += (double)bf16_lo(v[u][w]);
        acc[2 * w + 1] += (double)bf16_hi(v[u][w]);
      }
  }
  for (; t < t1; ++t) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p + (int64_t)t * sl);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += (double)bf16_lo(v[w]);
      acc[2 * w + 1] += (double)bf16_hi(v[w]);
    }
  }
  const double n = (double)(t1 - t0);
  double* o = out + (((int64_t)b * H + h) * nblk + blk) * D + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = acc[i] / n;
}

__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t u = __double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Orders this wave's LDS accesses (the histogram of a row is private to its
// wave, so no workgroup barrier is needed and waves may leave the radix
// loop at different passes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Chunk range [first, last] of the tokens [t0, t1) (t1 > t0).
__device__ __forceinline__ void chunk_span(int t0, int t1, int ar, int& first, int& last) {
  first = t0 / ar;
  last = (t1 - 1) / ar;
}

// Radix select from the top over 64-bit keys (8-bit digits, LDS histogram
// private to the wave; bit j of `valid` marks key j of the lane, NPL <= 32):
// on return the leading bits `pmask` of the kk-th
// largest valid key are `prefix`; every valid key above prefix on those bits
// is among the kk largest, and of the keys equal to it on those bits the
// first `remaining` in index order complete them (all of them when the loop
// stopped early because every candidate left in the chosen bin is kept).
// With every bit examined, prefix is the exact kk-th largest key.
template <int NPL, typename Key>
__device__ __forceinline__ void radix_select_desc(const Key (&key)[NPL], uint32_t valid, int kk, uint32_t* hist,
                                                  int lane, Key& prefix, Key& pmask, int& remaining) {
  constexpr int kBits = 8 * (int)sizeof(Key);
  for (int shift = kBits - 8; shift >= 0 && kk > 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const bool f = ((valid >> j) & 1u) && (key[j] & pmask) == prefix;
      if (shift < kBits - 16) {
        if (f) atomicAdd(&hist[(uint32_t)(key[j] >> shift) & 255u], 1u);
        continue;
      }
      const uint64_t fm = __ballot(f);
      if (fm) {
        const uint32_t dg = (uint32_t)(key[j] >> shift) & 255u;
        const int lead = __builtin_ctzll(fm);
        const uint32_t d0 = (uint32_t)__shfl((int)dg, lead);
        if (__ballot(f && dg != d0) == 0) {
          // one digit for every candidate of this chunk (the rule in the two
          // leading digits, sign and exponent): one update instead of 64
          // contended LDS atomics
          if (lane == lead) atomicAdd(&hist[d0], (uint32_t)__popcll(fm));
        } else if (f) {
          atomicAdd(&hist[dg], 1u);
        }
      }
    }
    wave_lds_sync();
    // lane covers bins 255-4*lane .. 252-4*lane, i.e. digits in descending order
    uint32_t cnt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt[i] = hist[255 - 4 * lane - i];
    const uint32_t s = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t up = (uint32_t)__shfl_up((int)incl, o);
      if (lane >= o) incl += up;
    }
    const uint64_t hit = __ballot(incl >= (uint32_t)remaining);
    const int src = hit ? (__builtin_ctzll(hit)) : 63;
    uint32_t above = incl - s;
    int digit = 255 - 4 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (above + cnt[i] >= (uint32_t)remaining) {
        digit = 255 - 4 * lane - i;
        break;
      }
      above += cnt[i];
    }
    uint32_t in_bin = 0;  // candidates in the chosen bin
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (digit == 255 - 4 * lane - i) in_bin = cnt[i];
    digit = __shfl(digit, src);
    above = (uint32_t)__shfl((int)above, src);
    in_bin = (uint32_t)__shfl((int)in_bin, src);
    remaining -= (int)above;
    prefix |= (Key)digit << shift;
    pmask |= (Key)0xFF << shift;
    wave_lds_sync();
    // every candidate left in the chosen bin is kept: the bits below do not
    // change the selection (wave-uniform exit)
    if (in_bin == (uint32_t)remaining) break;
  }

}

template <int NPL>  // scores per lane (row length <= 64 * NPL)
__global__ __launch_bounds__(256) void topk_rows_kernel(const double* __restrict__ S, int64_t n_rows, int C, int k,
                                                        MapRule rule, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[4][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  const bool row_ok = row < n_rows;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // Causal window: key block c may be kept by query block qb when its
  // chunks [ck0, ck1] meet [cq0 - W + 1, cq1], the chunks the queries of qb
  // see (no lower limit for W = 0); without a window every block is allowed.
  const int qb = (int)(row % rule.Nq);
  int cq0 = 0, cq1 = 0;
  if (rule.ar_tokens < rule.L) chunk_span(qb * rule.bq, min(rule.L, (qb + 1) * rule.bq), rule.ar_tokens, cq0, cq1);
  const int lo_chunk = rule.ar_window > 0 ? cq0 - rule.ar_window + 1 : -1;
  const double* Srow = S + (row % rule.s_rows) * (int64_t)C;
  uint64_t key[NPL];
  uint32_t valid = 0;
  int n_ok = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int c = j * 64 + lane;
    bool ok = row_ok && c < C;
    if (ok && rule.ar_tokens < rule.L) {
      int ck0, ck1;
      chunk_span(c * rule.bk, min(rule.L, (c + 1) * rule.bk), rule.ar_tokens, ck0, ck1);
      ok = ck0 <= cq1 && ck1 >= lo_chunk;
    }
    valid |= (ok ? 1u : 0u) << j;
    key[j] = ok ? order_key(Srow[c]) : 0ull;
    n_ok += __popcll(__ballot(ok));
  }
  // fewer allowed blocks than k: all of them are kept, the rest is -1
  const int kk = min(k, n_ok);

  uint64_t prefix = 0, pmask = 0;
  int remaining = kk;
  radix_select_desc<NPL>(key, valid, kk, hist[wv], lane, prefix, pmask, remaining);

  if (!row_ok) return;
  // keys whose leading bits (pmask) exceed the prefix are kept, and of those
  // equal to it on those bits the first `remaining` in index order (all of
  // them when the loop ended early); with every bit examined, prefix is the
  // exact k-th largest key
  for (int rep = 0; rep < rule.n_rep; ++rep) {
    int taken = 0, ties = 0;
    int32_t* out = idx + rep * rule.rep_stride + row * k;
    if (kk > 0) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const uint64_t km = key[j] & pmask;
        const bool vj = (valid >> j) & 1u;
        const bool gt = vj && km > prefix;
        const bool eq = vj && km == prefix;
        const uint64_t eqm = __ballot(eq);
        const bool take = gt || (eq && ties + __popcll(eqm & lt_mask) < remaining);
        const uint64_t tm = __ballot(take);
        if (take) out[taken + __popcll(tm & lt_mask)] = j * 64 + lane;
        taken += __popcll(tm);
        ties += __popcll(eqm);
      }
    }
    for (int i = kk + lane; i < k; i += 64) out[i] = -1;
  }
}

// ---------------------------------------------------------------------------
// Scores and exact top-k in one kernel, without the score matrix.
//
// kmean_split_kernel first writes each float64 key-block mean as bf16 hi +
// lo parts (x ~= hi + lo to about 2^-18 of x). A workgroup of 16 waves then
// takes 16 query-block rows of one (batch, head) (8 for the longest rows)
// and every key block.
// Phase 1: the approximate scores S' = qbar . kbar on 16x16x32 bf16 MFMAs
// (three products per pair of split operands, f32 accumulation), kept in
// LDS as f32. Each product term is exact in f32, so |S - S'| <=
// (3 * 2^-18 + 3 d 2^-24) sum_d |qbar_d kbar_d|, which the kernel bounds by
// delta = 2^-12 |qbar_b| max_c |kbar_c| (Cauchy-Schwarz; d <= 128; the
// largest norm is formed from the split parts in f32 and raised by 2^-10).
// Phase 2, one wave per row: sigma = the k-th largest S' (radix select on
// the order-preserving 32-bit images). A block with S' > sigma + 2 delta is
// kept for certain (fewer than k blocks can reach its score), one with
// S' < sigma - 2 delta is dropped for certain (k blocks beat it); only the
// few in between (five per row on average at 720P) get their exact float64
// score, sixteen lanes each, and a radix select over those exact keys fills
// the remaining places, equal scores going to the lower block index. The
// kept set is therefore exactly the top-k of the float64 scores. Rows are
// written ascending; the causal-window rule and -1 padding are those of
// topk_rows_kernel.
// ---------------------------------------------------------------------------
constexpr int kSelWaves = 16;
// query-block rows per workgroup: 16, or 8 for the longest rows, so that the
// approximate scores fit the LDS
__host__ __device__ constexpr int sel_rows(int npl) { return npl <= 24 ? 16 : 8; }

__device__ __forceinline__ uint32_t order_key32(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// Split 8 float64 values into bf16 hi + lo MFMA operands (x ~= hi + lo to
// about 2^-18 of x) and add their squares to ss.
__device__ __forceinline__ void split_f64x8(const double* v, bf16x8& hi, bf16x8& lo, double& ss) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double x = v[e];
    const __bf16 h = (__bf16)(float)x;
    hi[e] = h;
    lo[e] = (__bf16)(float)(x - (double)(float)h);
    ss = fma(x, x, ss);
  }
}

// The key-block means as the A operands of the approximate scores: bf16 hi
// and lo parts of each float64 mean (x ~= hi + lo to about 2^-18 of x).
// One thread per 8 channels of one key block.
__global__ __launch_bounds__(256) void kmean_split_kernel(const double* __restrict__ kmean, int64_t n_vec,
                                                          uint16_t* __restrict__ khi, uint16_t* __restrict__ klo) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_vec) return;
  double v[8], ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = kmean[8 * t + e];
  bf16x8 hi, lo;
  split_f64x8(v, hi, lo, ss);
  *reinterpret_cast<bf16x8*>(khi + 8 * t) = hi;
  *reinterpret_cast<bf16x8*>(klo + 8 * t) = lo;
}

template <int D, int NPL>
__global__ __launch_bounds__(64 * kSelWaves) void select_topk_kernel(const double* __restrict__ qmean,
                                                                     const double* __restrict__ kmean,
                                                                     const uint16_t* __restrict__ khi,
                                                                     const uint16_t* __restrict__ klo, int k,
                                                                     MapRule rule, int Nk,
                                                                     int32_t* __restrict__ idx) {
  constexpr int R = sel_rows(NPL), NW = kSelWaves;
  constexpr int NKP = 64 * NPL + 4;  // row pitch of the approximate scores, in floats
  __shared__ __attribute__((aligned(16))) float Sa[R * NKP];
  __shared__ uint32_t hist[NW][256];
  __shared__ int lst_c[NW][64];         // undecided blocks of the row, in index order
  __shared__ uint64_t lst_key[NW][64];  // their exact keys
  __shared__ uint32_t chosen[NW][64];   // bit c % 32 of word c / 32: undecided block c is kept
  __shared__ float kmax2[NW];
  __shared__ double qn2[R];
  const int Nq = rule.Nq;
  const int64_t bh = blockIdx.y;
  const int r0 = blockIdx.x * R;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kg = lane >> 4;
  const double* Qm = qmean + bh * (int64_t)Nq * D;
  const double* Km = kmean + bh * (int64_t)Nk * D;

  // B operands: the query-block means, row l16, d = 32 s + 8 kg .. + 7
  bf16x8 qh[D / 32], ql[D / 32];
  {
    const int row = r0 + l16;
    double ss = 0.0;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      double v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = row < Nq ? Qm[(int64_t)row * D + 32 * s + 8 * kg + e] : 0.0;
      split_f64x8(v, qh[s], ql[s], ss);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (wv == 0 && lane < 16) qn2[lane] = ss;
  }
  // S'^T tiles of 16 key blocks x 16 rows: A = the split key means (lane:
  // key l16, d = 32 s + 8 kg ..), accumulator lane: row l16, keys 4 kg ..
  // 4 kg + 3
  const uint16_t* Kh = khi + bh * (int64_t)Nk * D;
  const uint16_t* Kl = klo + bh * (int64_t)Nk * D;
  // (also the largest squared norm of the head's key means, from hi + lo in
  // f32: within 2^-16 of the float64 value)
  const int ntile = (Nk + 15) / 16;
  float kmx = 0.f;
  for (int t = wv; t < ntile; t += NW) {
    const int c = 16 * t + l16;
    f32x4 acc = {};
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const int64_t off = (int64_t)c * D + 32 * s + 8 * kg;
      const bf16x8 kh = c < Nk ? *reinterpret_cast<const bf16x8*>(Kh + off) : bf16x8{};
      const bf16x8 kl = c < Nk ? *reinterpret_cast<const bf16x8*>(Kl + off) : bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[s], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[s], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[s], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)kh[e] + (float)kl[e];
        ss = fmaf(x, x, ss);
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    kmx = fmaxf(kmx, ss);
    if (l16 < R) *reinterpret_cast<f32x4*>(Sa + l16 * NKP + 16 * t + 4 * kg) = acc;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, o));
  if (lane == 0) kmax2[wv] = kmx;
  __syncthreads();
  float km2 = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) km2 = fmaxf(km2, kmax2[w]);
  const double kmax = sqrt((double)km2) * (1.0 + 0x1p-10);

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int rr = wv; rr < R; rr += NW) {
    const int qb = r0 + rr;
    if (qb >= Nq) break;
    int cq0 = 0, cq1 = 0;
    if (rule.ar_tokens < rule.L) chunk_span(qb * rule.bq, min(rule.L, (qb + 1) * rule.bq), rule.ar_tokens, cq0, cq1);
    const int lo_chunk = rule.ar_window > 0 ? cq0 - rule.ar_window + 1 : -1;
    uint32_t akey[NPL];  // order-preserving images of the approximate scores
    uint32_t valid = 0;
    int n_ok = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int c = j * 64 + lane;
      bool ok = c < Nk;
      if (ok && rule.ar_tokens < rule.L) {
        int ck0, ck1;
        chunk_span(c * rule.bk, min(rule.L, (c + 1) * rule.bk), rule.ar_tokens, ck0, ck1);
        ok = ck0 <= cq1 && ck1 >= lo_chunk;
      }
      valid |= (ok ? 1u : 0u) << j;
      akey[j] = ok ? order_key32(Sa[rr * NKP + c]) : 0u;
      n_ok += __popcll(__ballot(ok));
    }
    const int kk = min(k, n_ok);
    int32_t* out = idx + (bh * Nq + qb) * (int64_t)k;
    uint32_t take_i = 0;  // bit j: block j * 64 + lane is kept
    if (kk > 0) {
      // sigma: the kk-th largest approximate score
      uint32_t pre = 0, pm = 0;
      int rem = kk;
      radix_select_desc<NPL>(akey, valid, kk, hist[wv], lane, pre, pm, rem);
      uint32_t smin = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (((valid >> j) & 1u) && (akey[j] & pm) == pre) smin = min(smin, akey[j]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) smin = min(smin, (uint32_t)__shfl_xor((int)smin, o));
      auto score_of = [](uint32_t k32) { return __uint_as_float((k32 >> 31) ? (k32 & 0x7FFFFFFFu) : ~k32); };
      const double sigma = (double)score_of(smin);
      const double delta = 0x1p-12 * sqrt(qn2[rr]) * kmax;
      const double hi_b = sigma + 2.0 * delta, lo_b = sigma - 2.0 * delta;
      uint32_t in_m = 0;  // bit j: undecided
      int n_i = 0, n_m = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const double sj = (double)score_of(akey[j]);
        const bool vj = (valid >> j) & 1u;
        const bool ti = vj && sj > hi_b;
        const bool mi = vj && !ti && sj >= lo_b;
        take_i |= (ti ? 1u : 0u) << j;
        in_m |= (mi ? 1u : 0u) << j;
        n_i += __popcll(__ballot(ti));
        n_m += __popcll(__ballot(mi));
      }
      const int need = kk - n_i;
      const double* qrow = Qm + (int64_t)qb * D;
      if (n_m <= 64) {
        // Fast path. The undecided blocks, listed in index order, get their
        // exact scores sixteen lanes each (lane part p sums d in
        // [p D/16, (p+1) D/16) in order, then a fixed tree over the sixteen
        // parts); one key per lane, and the best `need` of them are marked.
        int base = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const bool mj = (in_m >> j) & 1u;
          const uint64_t mm = __ballot(mj);
          if (mj) lst_c[wv][base + __popcll(mm & lt_mask)] = j * 64 + lane;
          base += __popcll(mm);
        }
        chosen[wv][lane] = 0u;
        wave_lds_sync();
        constexpr int DP = D / 16;
        const int e_in = lane >> 4, part = lane & 15;
        for (int g0 = 0; g0 < n_m; g0 += 4) {
          const int e = g0 + e_in;
          const int c = e < n_m ? lst_c[wv][e] : 0;
          const double* kp = Km + (int64_t)c * D + part * DP;
          const double* qp = qrow + part * DP;
          double kv[DP], qv[DP];
#pragma unroll
          for (int u = 0; u < DP; ++u) {
            kv[u] = kp[u];
            qv[u] = qp[u];
          }
          double acc = 0.0;
#pragma unroll
          for (int u = 0; u < DP; ++u) acc = fma(qv[u], kv[u], acc);
          acc += __shfl_xor(acc, 1);
          acc += __shfl_xor(acc, 2);
          acc += __shfl_xor(acc, 4);
          acc += __shfl_xor(acc, 8);
          if (part == 0 && e < n_m) lst_key[wv][e] = order_key(acc);
        }
        wave_lds_sync();
        uint64_t ek[1] = {lane < n_m ? lst_key[wv][lane] : 0ull};
        const uint32_t ev = lane < n_m ? 1u : 0u;
        uint64_t pre2 = 0, pm2 = 0;
        int rem2 = need;
        radix_select_desc<1>(ek, ev, need, hist[wv], lane, pre2, pm2, rem2);
        const uint64_t km = ek[0] & pm2;
        const bool eq = ev && km == pre2;
        const bool pick = (ev && km > pre2) || (eq && __popcll(__ballot(eq) & lt_mask) < rem2);
        if (pick) {
          const int c = lst_c[wv][lane];
          atomicOr(&chosen[wv][c >> 5], 1u << (c & 31));
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const int c = j * 64 + lane;
          if (((in_m >> j) & 1u) && ((chosen[wv][c >> 5] >> (c & 31)) & 1u)) take_i |= 1u << j;
        }
      } else {
        // Many undecided blocks (only near-constant inputs): each gets its
        // exact score in place (FMAs in order of d), then a radix select
        // over them fills the remaining places in index order.
        uint64_t key[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          key[j] = 0ull;
          const bool mj = (in_m >> j) & 1u;
          if (__ballot(mj) != 0 && mj) {
            const double* krow = Km + (int64_t)(j * 64 + lane) * D;
            double acc = 0.0;
#pragma nounroll
            for (int d = 0; d < D; ++d) acc = fma(qrow[d], krow[d], acc);
            key[j] = order_key(acc);
          }
        }
        uint64_t pre2 = 0, pm2 = 0;
        int rem2 = need;
        radix_select_desc<NPL>(key, in_m, need, hist[wv], lane, pre2, pm2, rem2);
        int ties = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const uint64_t km = key[j] & pm2;
          const bool mj = (in_m >> j) & 1u;
          const bool eq = mj && km == pre2;
          const uint64_t eqm = __ballot(eq);
          const bool take = (mj && km > pre2) || (eq && ties + __popcll(eqm & lt_mask) < rem2);
          take_i |= (take ? 1u : 0u) << j;
          ties += __popcll(eqm);
        }
      }
    }
    // output in index order
    int taken = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const bool take = (take_i >> j) & 1u;
      const uint64_t tm = __ballot(take);
      const int pos = taken + __popcll(tm & lt_mask);
      if (take && pos < kk) out[pos] = j * 64 + lane;
      taken += __popcll(tm);
    }
    for (int i = kk + lane; i < k; i += 64) out[i] = -1;
  }
}

// Centroid (t, h, w) of each block of bs raster tokens: exact integer sums
// of the coordinates, one float64 division each.
__global__ void block_centroids_kernel(int L, int bs, int n, int Hg, int Wg, double* __restrict__ cen) {
  const int blk = blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n) return;
  const int t0 = blk * bs, t1 = min(L, t0 + bs);
  const int hw = Hg * Wg;
  int64_t st = 0, sh = 0, sw = 0;
  for (int i = t0; i < t1; ++i) {
    st += i / hw;
    sh += (i / Wg) % Hg;
    sw += i % Wg;
  }
  const double cnt = (double)(t1 - t0);
  cen[3 * blk + 0] = (double)st / cnt;
  cen[3 * blk + 1] = (double)sh / cnt;
  cen[3 * blk + 2] = (double)sw / cnt;
}

// S[r][c] = -((dt*dt + dh*dh) + dw*dw) of the two centroids, rounded after
// every operation (no fused multiply-add), so the value is reproducible.
__global__ void fixed_scores_kernel(const double* __restrict__ cq, const double* __restrict__ ck, int Nq, int Nk,
                                    double* __restrict__ S) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)Nq * Nk) return;
  const int r = (int)(i / Nk), c = (int)(i - (int64_t)r * Nk);
  const double dt = cq[3 * r] - ck[3 * c];
  const double dh = cq[3 * r + 1] - ck[3 * c + 1];
  const double dw = cq[3 * r + 2] - ck[3 * c + 2];
  const double sq_t = dt * dt, sq_h = dh * dh, sq_w = dw * dw;
  S[i] = -((sq_t + sq_h) + sq_w);
}

hipError_t launch_pool_blocks(const uint16_t* X, int64_t sb, int64_t sl, int64_t sh, int B, int L, int H, int D,
                              int bs, double* out, hipStream_t stream) {
  const int nblk = (L + bs - 1) / bs;
  const int chunks = H * (D / 8);
  const dim3 grid(nblk, B, (chunks + 255) / 256);
  hipLaunchKernelGGL(pool_blocks_kernel, grid, dim3(256), 0, stream, X, sb, sl, sh, L, H, D, bs, nblk, out);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const double* S, int64_t n_rows, int C, int k, const MapRule& rule, int32_t* idx,
                            hipStream_t stream) {
  const int npl = (C + 63) / 64;
  const dim3 grid((unsigned)((n_rows + 3) / 4)), block(256);
#define SD_TOPK_CASE(N)                                                                          \
  if (npl <= N) {                                                                                \
    hipLaunchKernelGGL(topk_rows_kernel<N>, grid, block, 0, stream, S, n_rows, C, k, rule, idx); \
    return hipGetLastError();                                                                    \
  }
  SD_TOPK_CASE(1)
  SD_TOPK_CASE(2)
  SD_TOPK_CASE(4)
  SD_TOPK_CASE(8)
  SD_TOPK_CASE(12)
  SD_TOPK_CASE(16)
  SD_TOPK_CASE(20)
  SD_TOPK_CASE(24)
  SD_TOPK_CASE(32)
#undef SD_TOPK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_select_topk(const double* qmean, const double* kmean, int BH, int Nk, int D, int k,
                              const MapRule& rule, uint16_t* khi, uint16_t* klo, int32_t* idx,
                              hipStream_t stream) {
  const int64_t n_vec = (int64_t)BH * Nk * (D / 8);
  hipLaunchKernelGGL(kmean_split_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256), 0, stream, kmean, n_vec,
                     khi, klo);
  const int npl = (Nk + 63) / 64;
#define SD_SEL_CASE(DD, N)                                                                                     \
  if (D == DD && npl <= N) {                                                                                   \
    const dim3 grid((unsigned)((rule.Nq + sel_rows(N) - 1) / sel_rows(N)), (unsigned)BH), block(64 * kSelWaves); \
    hipLaunchKernelGGL((select_topk_kernel<DD, N>), grid, block, 0, stream, qmean, kmean, khi, klo, k, rule, Nk, \
                       idx);                                                                                   \
    return hipGetLastError();                                                                                  \
  }
  SD_SEL_CASE(128, 4)
  SD_SEL_CASE(128, 8)
  SD_SEL_CASE(128, 12)
  SD_SEL_CASE(128, 16)
  SD_SEL_CASE(128, 20)
  SD_SEL_CASE(128, 24)
  SD_SEL_CASE(128, 32)
  SD_SEL_CASE(64, 4)
  SD_SEL_CASE(64, 8)
  SD_SEL_CASE(64, 12)
  SD_SEL_CASE(64, 16)
  SD_SEL_CASE(64, 20)
  SD_SEL_CASE(64, 24)
  SD_SEL_CASE(64, 32)
#undef SD_SEL_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fixed_scores(int L, int Nq, int Nk, int bq, int bk, int Hg, int Wg, double* cq, double* ck,
                               double* S, hipStream_t stream) {
  hipLaunchKernelGGL(block_centroids_kernel, dim3((Nq + 255) / 256), dim3(256), 0, stream, L, bq, Nq, Hg, Wg, cq);
  hipLaunchKernelGGL(block_centroids_kernel, dim3((Nk + 255) / 256), dim3(256), 0, stream, L, bk, Nk, Hg, Wg, ck);
  const int64_t n = (int64_t)Nq * Nk;
  hipLaunchKernelGGL(fixed_scores_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, cq, ck, Nq, Nk,
                     S);
  return hipGetLastError();
}

}  // namespace sd
