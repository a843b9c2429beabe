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
  // 8 rows in flight per thread (the rows are read once: non-temporal)
  int t = t0;
  for (; t + 8 <= t1; t += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + (int64_t)(t + u) * sl));
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += (double)bf16_lo(v[u][w]);
        acc[2 * w + 1] += (double)bf16_hi(v[u][w]);
      }
  }
  for (; t < t1; ++t) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + (int64_t)t * sl));
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
template <int NPL, typename Key, int kBits = 8 * (int)sizeof(Key)>
__device__ __forceinline__ void radix_select_desc(const Key (&key)[NPL], uint32_t valid, int kk, uint32_t* hist,
                                                  int lane, Key& prefix, Key& pmask, int& remaining) {
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
// lo parts (x ~= hi + lo to about 2^-18 of x) and its squared norm. A
// workgroup of 16 waves then takes 32 query-block rows of one (batch, head)
// (16 for the longest rows) and every key block.
// Phase 1: the approximate scores S' = qbar . kbar on 16x16x32 bf16 MFMAs
// (three products per pair of split operands, f32 accumulation). Each
// product term is exact in f32, so |S - S'| <= (3 * 2^-18 + 3 d 2^-24)
// sum_d |qbar_d kbar_d| <= 2^-14.8 |qbar_b| kmax (Cauchy-Schwarz, d <= 128,
// kmax = the largest key-block norm of the head). They are kept in LDS as
// 16-bit fixed point of the normalised score S' / (|qbar_b| kmax) (|.| <=
// 1 + 2^-12), 2^14 steps per unit: rounding adds 2^-15. So every stored
// value is within Delta = 2^-12 (in normalised units, 4 steps) of the exact
// normalised score, with room for a coarser MFMA accumulation.
// Phase 2, one wave per row: sigma = the k-th largest stored value (a
// bitwise search on ballot counts of the 16-bit keys). A block more than 2 Delta (8 steps) above
// sigma is kept for certain (fewer than k blocks can reach its score), one
// more than 2 Delta below is dropped for certain (k blocks beat it); only
// the few in between (about five per row at 720P) get their exact float64
// score, sixteen lanes each, and are ranked by it, equal scores going to
// the lower block index. The kept set is therefore exactly the top-k of the
// float64 scores. Rows are written ascending; the causal-window rule and -1
// padding are those of topk_rows_kernel.
// ---------------------------------------------------------------------------
constexpr int kSelWaves = 16;
// query-block rows per workgroup: 32, or 16 for the longest rows, so that
// the approximate scores fit the LDS
__host__ __device__ constexpr int sel_rows(int npl) { return npl <= 24 ? 32 : 16; }
constexpr float kSelSteps = 16384.f;  // fixed-point steps per normalised unit
constexpr int kSelBand = 8;           // 2 Delta in steps

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
// and lo parts of each float64 mean (x ~= hi + lo to about 2^-18 of x), and
// the squared norm of each mean (float64). One thread per 8 channels of one
// key block; the cpk = d / 8 threads of a block are adjacent lanes of a wave.
__global__ __launch_bounds__(256) void kmean_split_kernel(const double* __restrict__ kmean, int64_t n_vec, int cpk,
                                                          uint16_t* __restrict__ khi, uint16_t* __restrict__ klo,
                                                          double* __restrict__ knorm2) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = t < n_vec;
  double v[8], ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = ok ? kmean[8 * t + e] : 0.0;
  bf16x8 hi, lo;
  split_f64x8(v, hi, lo, ss);
  for (int o = 1; o < cpk; o <<= 1) ss += __shfl_xor(ss, o);
  if (!ok) return;
  *reinterpret_cast<bf16x8*>(khi + 8 * t) = hi;
  *reinterpret_cast<bf16x8*>(klo + 8 * t) = lo;
  if ((t & (cpk - 1)) == 0) knorm2[t / cpk] = ss;
}

template <int D, int NPL>
__global__ __launch_bounds__(64 * kSelWaves) void select_topk_kernel(const double* __restrict__ qmean,
                                                                     const double* __restrict__ kmean,
                                                                     const uint16_t* __restrict__ khi,
                                                                     const uint16_t* __restrict__ klo,
                                                                     const double* __restrict__ knorm2, int k,
                                                                     MapRule rule, int Nk,
                                                                     int32_t* __restrict__ idx) {
  constexpr int R = sel_rows(NPL), RG = R / 16, NW = kSelWaves;
  constexpr int NKP = 64 * NPL + 8;  // row pitch of the stored scores (int16)
  __shared__ __attribute__((aligned(16))) int16_t Sa[R * NKP];
  __shared__ uint32_t hist[NW][256];
  __shared__ int lst_c[NW][64];         // undecided blocks of the row, in index order
  __shared__ uint64_t lst_key[NW][64];  // their exact keys
  __shared__ uint32_t lst_pk[NW][128];  // compacted candidates: key << 16 | block
  __shared__ double red[NW];
  // the query-block means as split B operands: [row group][d step][lane]
  __shared__ bf16x8 Qs_hi[RG][D / 32][64], Qs_lo[RG][D / 32][64];
  __shared__ double qn2s[R];
  const int Nq = rule.Nq;
  const int64_t bh = blockIdx.y;
  const int r0 = blockIdx.x * R;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kg = lane >> 4;
  const double* Qm = qmean + bh * (int64_t)Nq * D;
  const double* Km = kmean + bh * (int64_t)Nk * D;

  // kmax: the largest key-block norm of the head
  {
    double mx = 0.0;
    for (int c = threadIdx.x; c < Nk; c += 64 * NW) mx = fmax(mx, knorm2[bh * Nk + c]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wv] = mx;
  }
  // B operands (wave rg < RG): the query-block means of rows r0 + 16 rg +
  // l16, d = 32 s + 8 kg .. + 7, split, and each row's squared norm
  if (wv < RG) {
    const int row = r0 + 16 * wv + l16;
    double ss = 0.0;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      double v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = row < Nq ? Qm[(int64_t)row * D + 32 * s + 8 * kg + e] : 0.0;
      bf16x8 hi, lo;
      split_f64x8(v, hi, lo, ss);
      Qs_hi[wv][s][lane] = hi;
      Qs_lo[wv][s][lane] = lo;
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 16) qn2s[16 * wv + lane] = ss;
  }
  __syncthreads();
  double km2 = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) km2 = fmax(km2, red[w]);
  // raised by 2^-30: the float64 norms are within far less of the exact ones
  const double kmax = sqrt(km2) * (1.0 + 0x1p-30);
  // the fixed-point scale of each of the lane's rows: 2^14 / (|qbar| kmax)
  float fscale[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const double nrm = sqrt(qn2s[16 * rg + l16]) * kmax;
    fscale[rg] = nrm > 0.0 ? (float)((double)kSelSteps / nrm) : 0.f;
  }

  // Phase 1. S'^T tiles of 16 key blocks x 16 rows: A = the split key means
  // (lane: key l16, d = 32 s + 8 kg ..), accumulator lane: row l16, keys
  // 4 kg .. 4 kg + 3.
  const uint16_t* Kh = khi + bh * (int64_t)Nk * D;
  const uint16_t* Kl = klo + bh * (int64_t)Nk * D;
  const int ntile = (Nk + 15) / 16;
  auto load_tile = [&](int t, bf16x8 (&kh)[D / 32], bf16x8 (&kl)[D / 32]) __attribute__((always_inline)) {
    const int c = 16 * t + l16;
    const bool ok = t < ntile && c < Nk;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const int64_t off = (int64_t)c * D + 32 * s + 8 * kg;
      kh[s] = ok ? *reinterpret_cast<const bf16x8*>(Kh + off) : bf16x8{};
      kl[s] = ok ? *reinterpret_cast<const bf16x8*>(Kl + off) : bf16x8{};
    }
  };
  for (int t = wv; t < ntile; t += NW) {
    bf16x8 ch[D / 32], cl[D / 32];
    load_tile(t, ch, cl);
    f32x4 acc[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const bf16x8 bh_ = Qs_hi[rg][s][lane], bl_ = Qs_lo[rg][s][lane];
        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch[s], bh_, acc[rg], 0, 0, 0);
        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch[s], bl_, acc[rg], 0, 0, 0);
        acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cl[s], bh_, acc[rg], 0, 0, 0);
      }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      int16_t q4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = fminf(fmaxf(acc[rg][e] * fscale[rg], -32767.f), 32767.f);
        q4[e] = (int16_t)__float2int_rn(x);
      }
      *reinterpret_cast<uint64_t*>(Sa + (16 * rg + l16) * NKP + 16 * t + 4 * kg) =
          __builtin_bit_cast(uint64_t, q4);
    }
  }
  __syncthreads();

  // Phase 2, one wave per row.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma nounroll
  for (int rr = wv; rr < R; rr += NW) {
    const int qb = r0 + rr;
    if (qb >= Nq) break;
    int cq0 = 0, cq1 = 0;
    if (rule.ar_tokens < rule.L) chunk_span(qb * rule.bq, min(rule.L, (qb + 1) * rule.bq), rule.ar_tokens, cq0, cq1);
    const int lo_chunk = rule.ar_window > 0 ? cq0 - rule.ar_window + 1 : -1;
    uint32_t akey[NPL];  // order-preserving 16-bit images of the stored scores
    uint32_t valid = 0;
    int n_ok = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      int c = j * 64 + lane;
      // (kept opaque: recomputing the window test per row is cheaper than
      // holding all NPL of its results in registers across the rows)
      asm volatile("" : "+v"(c));
      bool ok = c < Nk;
      if (ok && rule.ar_tokens < rule.L) {
        int ck0, ck1;
        chunk_span(c * rule.bk, min(rule.L, (c + 1) * rule.bk), rule.ar_tokens, ck0, ck1);
        ok = ck0 <= cq1 && ck1 >= lo_chunk;
      }
      valid |= (ok ? 1u : 0u) << j;
      akey[j] = ok ? (uint32_t)((int)Sa[rr * NKP + c] + 32768) : 0u;
      n_ok += __popcll(__ballot(ok));
    }
    const int kk = min(k, n_ok);
    int32_t* out = idx + (bh * Nq + qb) * (int64_t)k;
    const double* qrow = Qm + (int64_t)qb * D;

    // The undecided blocks listed in lst_c[wv][0, n_m) (n_m <= 64, index
    // order) get their exact scores sixteen lanes each (lane part p sums d
    // in [p D/16, (p+1) D/16) in order, then a fixed tree over the sixteen
    // parts) and are ranked against each other (higher score first, the
    // lower index first among equal scores). Returns the mask of list
    // entries among the best `need`.
    auto exact_pick = [&](int n_m, int need) __attribute__((always_inline)) -> uint64_t {
      constexpr int DP = D / 16;
      const int e_in = lane >> 4, part = lane & 15;
      wave_lds_sync();
      // the query part is the same for every block; two groups of four
      // blocks go per pass, their loads issued together
      double qv[DP];
#pragma unroll
      for (int u = 0; u < DP; ++u) qv[u] = qrow[part * DP + u];
      for (int g0 = 0; g0 < n_m; g0 += 8) {
        int e[2], c[2];
        double kv[2][DP];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          e[h] = g0 + 4 * h + e_in;
          c[h] = e[h] < n_m ? lst_c[wv][e[h]] : 0;
#pragma unroll
          for (int u = 0; u < DP; ++u) kv[h][u] = Km[(int64_t)c[h] * D + part * DP + u];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          double acc = 0.0;
#pragma unroll
          for (int u = 0; u < DP; ++u) acc = fma(qv[u], kv[h][u], acc);
          acc += __shfl_xor(acc, 1);
          acc += __shfl_xor(acc, 2);
          acc += __shfl_xor(acc, 4);
          acc += __shfl_xor(acc, 8);
          if (part == 0 && e[h] < n_m) lst_key[wv][e[h]] = order_key(acc);
        }
      }
      wave_lds_sync();
      const uint64_t mine = lane < n_m ? lst_key[wv][lane] : 0ull;
      const uint32_t mine_lo = (uint32_t)mine, mine_hi = (uint32_t)(mine >> 32);
      int rank = 0;
      for (int i = 0; i < n_m; ++i) {
        const uint64_t other = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mine_hi, i) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)mine_lo, i);
        rank += (other > mine || (other == mine && i < lane)) ? 1 : 0;
      }
      return __ballot(lane < n_m && rank < need);
    };

    // Fast path: a lower bound on sigma is the kk-th largest of the lanes'
    // maxima (each is a key, so at least kk keys reach it). Every block that
    // can be kept or undecided scores at least that bound minus the band;
    // at 720P about 50 blocks a row do. With at most 128 of them they are
    // compacted (index order) to two per lane, and sigma, the decisions and
    // the output come from those alone.
    bool done = false;
    if (kk > 0 && kk <= 64) {
      uint32_t lmax = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) lmax = max(lmax, akey[j]);  // invalid keys are 0
      uint32_t lb = 0;
#pragma unroll
      for (int b = 15; b >= 0; --b) {
        const uint32_t t = lb | (1u << b);
        if (__popcll(__ballot(lmax >= t)) >= kk) lb = t;
      }
      const uint32_t floor_key = lb > (uint32_t)kSelBand + 1u ? lb - (uint32_t)kSelBand : 1u;
      int n_c = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) n_c += __popcll(__ballot(akey[j] >= floor_key));
      if (n_c <= 128) {
        int base = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const bool f = akey[j] >= floor_key;
          const uint64_t fm = __ballot(f);
          int c = j * 64 + lane;
          asm volatile("" : "+v"(c));
          if (f) lst_pk[wv][base + __popcll(fm & lt_mask)] = (akey[j] << 16) | (uint32_t)c;
          base += __popcll(fm);
        }
        wave_lds_sync();
        uint32_t ck[2], cc[2];  // candidate 64 x + lane: key (0: none), block
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t pk = 64 * x + lane < n_c ? lst_pk[wv][64 * x + lane] : 0u;
          ck[x] = pk >> 16;
          cc[x] = pk & 0xFFFFu;
        }
        uint32_t sig_u = 0;  // the kk-th largest key (sigma >= lb >= floor_key)
#pragma unroll
        for (int b = 15; b >= 0; --b) {
          const uint32_t t = sig_u | (1u << b);
          if (__popcll(__ballot(ck[0] >= t)) + __popcll(__ballot(ck[1] >= t)) >= kk) sig_u = t;
        }
        const int sig = (int)sig_u;
        bool ti[2], mi[2];
        uint64_t tm[2], mm[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int v = (int)ck[x];
          ti[x] = v > 0 && v > sig + kSelBand;
          mi[x] = v > 0 && !ti[x] && v >= sig - kSelBand;
          tm[x] = __ballot(ti[x]);
          mm[x] = __ballot(mi[x]);
        }
        const int n_m = __popcll(mm[0]) + __popcll(mm[1]);
        if (n_m <= 64) {
          const int need = kk - (__popcll(tm[0]) + __popcll(tm[1]));
          int me[2];  // the candidate's entry in the undecided list
          me[0] = __popcll(mm[0] & lt_mask);
          me[1] = __popcll(mm[0]) + __popcll(mm[1] & lt_mask);
#pragma unroll
          for (int x = 0; x < 2; ++x)
            if (mi[x]) lst_c[wv][me[x]] = (int)cc[x];
          const uint64_t pick = exact_pick(n_m, need);
          int taken = 0;
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const bool keep = ti[x] || (mi[x] && ((pick >> me[x]) & 1ull));
            const uint64_t km = __ballot(keep);
            const int pos = taken + __popcll(km & lt_mask);
            if (keep && pos < kk) out[pos] = (int)cc[x];
            taken += __popcll(km);
          }
          for (int i = kk + lane; i < k; i += 64) out[i] = -1;
          done = true;
        }
      }
    }
    if (done) continue;

    uint32_t take_i = 0;  // bit j: block j * 64 + lane is kept
    if (kk > 0) {
      // sigma: the kk-th largest stored value, the largest t with at least
      // kk keys >= t, found bit by bit from the top with ballot counts (no
      // LDS; invalid keys are 0 and valid ones at least 1)
      uint32_t sig_u = 0;
#pragma unroll
      for (int b = 15; b >= 0; --b) {
        const uint32_t t = sig_u | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) cnt += __popcll(__ballot(akey[j] >= t));
        if (cnt >= kk) sig_u = t;
      }
      const int sig = (int)sig_u;
      uint32_t in_m = 0;  // bit j: undecided
      int n_i = 0, n_m = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int v = (int)akey[j];
        const bool vj = (valid >> j) & 1u;
        const bool ti = vj && v > sig + kSelBand;
        const bool mi = vj && !ti && v >= sig - kSelBand;
        take_i |= (ti ? 1u : 0u) << j;
        in_m |= (mi ? 1u : 0u) << j;
        n_i += __popcll(__ballot(ti));
        n_m += __popcll(__ballot(mi));
      }
      const int need = kk - n_i;
      if (n_m <= 64) {
        int base = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const bool mj = (in_m >> j) & 1u;
          const uint64_t mm = __ballot(mj);
          int c = j * 64 + lane;
          asm volatile("" : "+v"(c));
          if (mj) lst_c[wv][base + __popcll(mm & lt_mask)] = c;
          base += __popcll(mm);
        }
        const uint64_t pick = exact_pick(n_m, need);
        base = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const bool mj = (in_m >> j) & 1u;
          const uint64_t mm = __ballot(mj);
          if (mj && ((pick >> (base + __popcll(mm & lt_mask))) & 1ull)) take_i |= 1u << j;
          base += __popcll(mm);
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
                              const MapRule& rule, uint16_t* khi, uint16_t* klo, double* knorm2, int32_t* idx,
                              hipStream_t stream) {
  const int64_t n_vec = (int64_t)BH * Nk * (D / 8);
  hipLaunchKernelGGL(kmean_split_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256), 0, stream, kmean, n_vec,
                     D / 8, khi, klo, knorm2);
  const int npl = (Nk + 63) / 64;
#define SD_SEL_CASE(DD, N)                                                                                     \
  if (D == DD && npl <= N) {                                                                                   \
    const dim3 grid((unsigned)((rule.Nq + sel_rows(N) - 1) / sel_rows(N)), (unsigned)BH), block(64 * kSelWaves); \
    hipLaunchKernelGGL((select_topk_kernel<DD, N>), grid, block, 0, stream, qmean, kmean, khi, klo, knorm2, k,  \
                       rule, Nk, idx);                                                                         \
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
