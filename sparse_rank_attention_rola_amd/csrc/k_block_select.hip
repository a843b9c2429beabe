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
//  block_scores_kernel S[b, h] = qmean . kmean^T as a 128x128-tiled f64 GEMM
//                      on the vector ALUs (8x8 register blocking, LDS panels).
//  fixed_scores_kernel the fixed spatio-temporal pattern (same section: a
//                      fixed pattern may replace the scored selection):
//                      minus the squared distance of the block centroids in
//                      latent (t, h, w) coordinates.
//  topk_rows_kernel    one wavefront per score row: a radix select on 8-bit
//                      digits of the order-preserving 64-bit image of the
//                      scores, from the top, finds the k-th largest score
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

// S[bh][r][c] = sum_d A[bh][r][d] * Bm[bh][c][d]   (A: [R, D], Bm: [C, D]).
// 128 x 128 output tile per workgroup; thread (tx, ty) of a 16 x 16 grid
// owns 8 rows and 8 columns in adjacent pairs: per 8 x 16-byte LDS reads it
// issues 64 float64 FMAs, each output summed over d in order. The d-loop
// goes in steps of 16 through k-major LDS panels.
__global__ __launch_bounds__(256) void block_scores_kernel(const double* __restrict__ A, const double* __restrict__ Bm,
                                                           int R, int C, int D, double* __restrict__ S) {
  constexpr int TM = 128, TK = 16;
  constexpr int TP = TM + 2;  // panel row: 16-byte aligned, loader writes 2-way at most
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  __shared__ __attribute__((aligned(16))) double As[TK][TP];
  __shared__ __attribute__((aligned(16))) double Bs[TK][TP];
  const int bh = blockIdx.z;
  const int r0 = blockIdx.y * TM, c0 = blockIdx.x * TM;
  const double* Ab = A + (int64_t)bh * R * D;
  const double* Bb = Bm + (int64_t)bh * C * D;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  // thread (ty, tx) owns rows 2 ty + 32 i + {0, 1} and columns
  // 2 tx + 32 j + {0, 1} (i, j < 4): each pair is one 16-byte LDS read
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  // loader: 128 rows x 16 d per panel = 2048 values, 8 per thread: row lr,
  // d = lk .. lk + 7 (64 contiguous bytes of the row)
  const int lr = tid >> 1, lk = (tid & 1) * 8;
  const bool a_ok = r0 + lr < R, b_ok = c0 + lr < C;
  const double* ap = Ab + (int64_t)(a_ok ? r0 + lr : 0) * D + lk;
  const double* bp = Bb + (int64_t)(b_ok ? c0 + lr : 0) * D + lk;
  double av[8], bv[8];
  auto load_panel = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = a_ok ? ap[k0 + i] : 0.0;
      bv[i] = b_ok ? bp[k0 + i] : 0.0;
    }
  };
  load_panel(0);
  for (int k0 = 0; k0 < D; k0 += TK) {
    __syncthreads();  // the previous panel's readers are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      As[lk + i][lr] = av[i];
      Bs[lk + i][lr] = bv[i];
    }
    __syncthreads();
    if (k0 + TK < D) load_panel(k0 + TK);  // in flight during this panel's FMAs
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      f64x2 a2[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a2[i] = *reinterpret_cast<const f64x2*>(&As[kk][2 * ty + 32 * i]);
        b2[i] = *reinterpret_cast<const f64x2*>(&Bs[kk][2 * tx + 32 * i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fma(a2[i >> 1][i & 1], b2[j >> 1][j & 1], acc[i][j]);
    }
  }
  double* Sb = S + (int64_t)bh * R * C;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 2 * ty + 32 * (i >> 1) + (i & 1);
    if (r >= R) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + 2 * tx + 32 * (j >> 1) + (j & 1);
      if (c < C) Sb[(int64_t)r * C + c] = acc[i][j];
    }
  }
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
  bool valid[NPL];
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
    valid[j] = ok;
    key[j] = ok ? order_key(Srow[c]) : 0ull;
    n_ok += __popcll(__ballot(ok));
  }
  // fewer allowed blocks than k: all of them are kept, the rest is -1
  const int kk = min(k, n_ok);

  uint64_t prefix = 0, pmask = 0;
  int remaining = kk;
  for (int shift = 56; shift >= 0 && kk > 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[wv][lane + 64 * i] = 0;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const bool f = valid[j] && (key[j] & pmask) == prefix;
      if (shift < 48) {
        if (f) atomicAdd(&hist[wv][(uint32_t)(key[j] >> shift) & 255u], 1u);
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
          if (lane == lead) atomicAdd(&hist[wv][d0], (uint32_t)__popcll(fm));
        } else if (f) {
          atomicAdd(&hist[wv][dg], 1u);
        }
      }
    }
    wave_lds_sync();
    // lane covers bins 255-4*lane .. 252-4*lane, i.e. digits in descending order
    uint32_t cnt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt[i] = hist[wv][255 - 4 * lane - i];
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
    prefix |= (uint64_t)digit << shift;
    pmask |= 0xFFull << shift;
    wave_lds_sync();
    // every candidate left in the chosen bin is kept: the bits below do not
    // change the selection (wave-uniform exit)
    if (in_bin == (uint32_t)remaining) break;
  }

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
        const bool gt = valid[j] && km > prefix;
        const bool eq = valid[j] && km == prefix;
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

hipError_t launch_block_scores(const double* qmean, const double* kmean, int BH, int Nq, int Nk, int D, double* S,
                               hipStream_t stream) {
  const dim3 grid((Nk + 127) / 128, (Nq + 127) / 128, BH);
  hipLaunchKernelGGL(block_scores_kernel, grid, dim3(256), 0, stream, qmean, kmean, Nq, Nk, D, S);
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
