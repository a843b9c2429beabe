// Fused q/k producer of the attention block: RMSNorm of each token's
// projection row, then the backbone 3D RoPE on every head (robotworld.top
// SparkDiffusion write-up, section 2.1: the low-rank branch reuses the
// normalised q/k from before the backbone attention; kais-engine portability
// report, section 2.1: fused QKV + RoPE operator). On request it also emits
// the block means of the rotated Q and K that the block scores of the same
// section take, so that the prepare phase need not read Q and K again.
//
//   y_c  = x_c / sqrt(mean_c' x_c'^2 + eps) * gamma_c      (Qn / Kn, bf16)
//   out  = R(p) y per head, pairs (2m, 2m+1) rotated       (Q / K, bf16)
//   mean = sum over a block's tokens of out (as stored, bf16) / tokens, f64
//
// qk_norm_rope_kernel (no means): one wavefront streams one row (a token's
// q or k, H*d channels): lane l holds 16-byte chunks l, l + 64, ... of the
// row, all at the same offset inside a head (64 is a multiple of the d/8
// chunks of a head), so every lane rotates the same 4 channel pairs at
// every head and computes their cos/sin once per row. The workgroups are
// persistent: a wave handles rows of one tensor only and keeps that
// tensor's gamma in registers.
//
// qk_norm_rope_means_kernel: the block sums need every row of a block in
// one place, so one workgroup takes a segment of consecutive rows (a whole
// number of query and key blocks) of q or of k, and thread i owns the
// 16-byte chunks i + j * NTH (j < CPT; NTH = the workgroup's threads, a
// multiple of the d / 8 chunks of a head) of every row: 8 channels of one
// head each, all at the same offset inside their heads. Rows go in
// batches: each thread loads its chunks of the batch's rows; the cos/sin
// of every (row of the batch, pair of a head) are formed once for the
// workgroup (sincosf in f32 of position * theta) into LDS; the row sums of
// squares are reduced across the wave (lane exchanges) and across the
// waves (LDS); one barrier per batch. Then each thread normalises, rotates,
// stores, and adds the rounded rotated values to its float64 block sums,
// in token order as the pooling kernel's are; a block is written when its
// last token is done. The barrier per batch and the float64 sums cost
// about a third more time than the kernel without means (1.13 against
// 0.86 ms for q and k at 720P), about what the prepare phase saves by not
// pooling Q and K (0.29 ms).
#include "sd_device.h"
#include "sd_launch.h"

namespace sd {

namespace qkp {
constexpr int kMaxWaves = 16;
constexpr int kMaxSeg = 128;  // rows per segment
}  // namespace qkp

// NT: largest workgroup; MINW: waves per SIMD the registers must allow;
// CPT: chunks per thread; kBatch: rows per batch
template <int NT, int MINW, int CPT, int kBatch>
__global__ __launch_bounds__(NT, MINW) void qk_norm_rope_means_kernel(QkNormRopeArgs a) {
  using namespace qkp;
  const int tensor = blockIdx.z;  // 0: q, 1: k
  const int b = blockIdx.y;
  const int seg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int nth = blockDim.x;
  const int wv = tid >> 6, nwv = (nth + 63) >> 6;
  const int C = a.H * a.d;
  const int nch = C >> 3;
  const uint16_t* src = (tensor ? a.k : a.q) + (int64_t)b * a.L * a.ld_in;
  const uint16_t* gamma = tensor ? a.gamma_k : a.gamma_q;
  uint16_t* out_r = (tensor ? a.K : a.Q) + (int64_t)b * a.L * C;
  uint16_t* out_n = (tensor ? a.Kn : a.Qn) + (int64_t)b * a.L * C;
  double* mean = tensor ? a.kmean : a.qmean;
  const int bs = tensor ? a.block_k : a.block_q;  // block of the means
  __shared__ float red[2][kMaxWaves][kBatch];
  __shared__ float2 rtab[2][kBatch][kQkMaxPairs];  // (cos, sin) of [row of the batch][pair]

  bool on[CPT];
  int cc[CPT];
  u32x4 gv[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    on[j] = tid + j * nth < nch;
    cc[j] = on[j] ? tid + j * nth : 0;
    gv[j] = (on[j] && gamma) ? *reinterpret_cast<const u32x4*>(gamma + 8 * cc[j])
                             : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // 1.0
  }
  // the 4 channel pairs of these chunks inside their heads: dims 8 wc + 2 e
  const int wc = tid % (a.d >> 3);

  const int t0 = seg * a.seg_rows, t1 = min(a.L, t0 + a.seg_rows);
  const int np = a.d >> 1;
  double acc[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.0;
  int par = 0;
  for (int tb = t0; tb < t1; tb += kBatch) {
    u32x4 v[kBatch][CPT];
    float ss[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int t = tb + r;
#pragma unroll
      for (int j = 0; j < CPT; ++j)
        v[r][j] = (on[j] && t < t1)
                      ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)t * a.ld_in) + cc[j])
                      : u32x4{0, 0, 0, 0};
    }
    // the batch's cos/sin table (entry i: row i / np, pair i % np)
    for (int i = tid; i < kBatch * np; i += nth) {
      const int r = i / np, pi = i - r * np, t = tb + r;
      const int ax = a.pair_axis[pi];
      float cs = 1.f, sn = 0.f;
      if (ax >= 0 && t < t1) {
        const int p = ax == 0 ? t / (a.Hg * a.Wg) : ax == 1 ? (t / a.Wg) % a.Hg : t % a.Wg;
        sincosf((float)p * a.pair_theta[pi], &sn, &cs);
      }
      rtab[par][r][pi] = float2{cs, sn};
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_lo(v[r][j][w]), hi = bf16_hi(v[r][j][w]);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      ss[r] = s;
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < kBatch; ++r) red[par][wv][r] = ss[r];
    }
    __syncthreads();  // (red and rtab are double-buffered: one barrier per batch)
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      float s = 0.f;
      for (int w = 0; w < nwv; ++w) s += red[par][w][r];
      ss[r] = s;
    }
    const float2(*tab)[kQkMaxPairs] = rtab[par];
    par ^= 1;
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int t = tb + r;
      if (t >= t1) break;
      const float inv = 1.0f / sqrtf(ss[r] / (float)C + a.eps);
      const float2* cs = &tab[r][4 * wc];
      // the block ends with this token (or the sequence does)
      const bool blk_end = (t + 1) % bs == 0 || t + 1 == a.L;
      const int blk = t / bs;
      const double n_tok = (double)(t + 1 - blk * bs);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        u32x4 n, rot;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float y0 = bf16_lo(v[r][j][w]) * inv * bf16_lo(gv[j][w]);
          const float y1 = bf16_hi(v[r][j][w]) * inv * bf16_hi(gv[j][w]);
          n[w] = pack_bf16x2(y0, y1);
          rot[w] = pack_bf16x2(y0 * cs[w].x - y1 * cs[w].y, y0 * cs[w].y + y1 * cs[w].x);
        }
        if (on[j]) {
          __builtin_nontemporal_store(n, reinterpret_cast<u32x4*>(out_n + (int64_t)t * C) + cc[j]);
          __builtin_nontemporal_store(rot, reinterpret_cast<u32x4*>(out_r + (int64_t)t * C) + cc[j]);
        }
        if (mean) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[j][2 * w] += (double)bf16_lo(rot[w]);
            acc[j][2 * w + 1] += (double)bf16_hi(rot[w]);
          }
          if (blk_end) {
            if (on[j]) {
              const int hh = cc[j] / (a.d >> 3);
              double* o = mean + (((int64_t)b * a.H + hh) * ((a.L + bs - 1) / bs) + blk) * a.d + 8 * wc;
              if (t + 1 - blk * bs == bs) {
                // a whole block: dividing by the power of two bs is this product
                const double rn = tensor ? a.rcp_block_k : a.rcp_block_q;
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = acc[j][i] * rn;
              } else {
#pragma nounroll
                for (int i = 0; i < 8; ++i) o[i] = acc[j][i] / n_tok;
              }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = 0.0;
          }
        }
      }
      // one row at a time: keeps the batch's results from being held in
      // registers until the end of the batch
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// NJ: 16-byte chunks per lane (rows of up to 512 * NJ channels)
template <int NJ>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(QkNormRopeArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);  // global wave
  const int tensor = gw & 1;                             // 0: q, 1: k
  const int nw_t = gridDim.x * 2;                        // waves per tensor
  const int C = a.H * a.d;
  const int nch = C >> 3;
  const uint16_t* src = tensor ? a.k : a.q;
  const uint16_t* gamma = tensor ? a.gamma_k : a.gamma_q;
  uint16_t* out_r = tensor ? a.K : a.Q;
  uint16_t* out_n = tensor ? a.Kn : a.Qn;

  u32x4 gv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = j * 64 + lane;
    gv[j] = (c < nch && gamma) ? *reinterpret_cast<const u32x4*>(gamma + 8 * c)
                               : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // 1.0
  }
  // the 4 channel pairs of this lane inside a head: dims 8 w + 2 e
  const int wc = lane % (a.d >> 3);
  int p_axis[4];
  float p_theta[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pi = 4 * wc + e;
    p_axis[e] = a.pair_axis[pi];
    p_theta[e] = a.pair_theta[pi];
  }

  const int64_t rows = (int64_t)a.B * a.L;
  for (int64_t row = gw >> 1; row < rows; row += nw_t) {
    const int l = (int)(row % a.L);
    const int pos[3] = {l / (a.Hg * a.Wg), (l / a.Wg) % a.Hg, l % a.Wg};
    const u32x4* x = reinterpret_cast<const u32x4*>(src + row * a.ld_in);
    // keep gamma packed (bf16 pairs) in registers across rows instead of
    // letting the compiler hoist its float expansion
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(gv[j]));
    u32x4 v[NJ];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = j * 64 + lane;
      if (c < nch) {
        v[j] = __builtin_nontemporal_load(x + c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_lo(v[j][w]), hi = bf16_hi(v[j][w]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / (float)C + a.eps);
    float cs[4], sn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p_axis[e] >= 0) {
        sincosf((float)pos[p_axis[e]] * p_theta[e], &sn[e], &cs[e]);
      } else {
        cs[e] = 1.f;
        sn[e] = 0.f;
      }
    }
    u32x4* on = reinterpret_cast<u32x4*>(out_n + row * C);
    u32x4* orr = reinterpret_cast<u32x4*>(out_r + row * C);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = j * 64 + lane;
      if (c < nch) {
        u32x4 n, r;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float y0 = bf16_lo(v[j][w]) * inv * bf16_lo(gv[j][w]);
          const float y1 = bf16_hi(v[j][w]) * inv * bf16_hi(gv[j][w]);
          n[w] = pack_bf16x2(y0, y1);
          r[w] = pack_bf16x2(y0 * cs[w] - y1 * sn[w], y0 * sn[w] + y1 * cs[w]);
        }
        __builtin_nontemporal_store(n, on + c);
        __builtin_nontemporal_store(r, orr + c);
      }
    }
  }
}

hipError_t launch_qk_norm_rope(const QkNormRopeArgs& a, hipStream_t stream) {
  if (a.qmean || a.kmean) {
    // segments of consecutive rows, one thread per chunk, 4 rows per batch
    // (116 VGPRs: 4 waves per SIMD)
    const int nch = a.H * a.d / 8;
    const int threads = (nch + 63) / 64 * 64;
    if (threads > 1024 || a.seg_rows < 1 || a.seg_rows > qkp::kMaxSeg) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.L + a.seg_rows - 1) / a.seg_rows), (unsigned)a.B, 2);
    hipLaunchKernelGGL((qk_norm_rope_means_kernel<1024, 4, 1, 4>), grid, dim3(threads), 0, stream, a);
    return hipGetLastError();
  }
  // persistent: up to 3 workgroups of 4 waves per CU on 256 CUs, waves split
  // evenly between q and k
  const int64_t rows = (int64_t)a.B * a.L;
  const int64_t want = (rows + 1) / 2;  // workgroups if every wave took one row
  const dim3 grid((unsigned)(want < 768 ? (want > 0 ? want : 1) : 768));
  const int nj = (a.H * a.d / 8 + 63) / 64;
  if (nj <= 2)
    hipLaunchKernelGGL(qk_norm_rope_kernel<2>, grid, dim3(256), 0, stream, a);
  else if (nj <= 4)
    hipLaunchKernelGGL(qk_norm_rope_kernel<4>, grid, dim3(256), 0, stream, a);
  else if (nj <= 6)
    hipLaunchKernelGGL(qk_norm_rope_kernel<6>, grid, dim3(256), 0, stream, a);
  else if (nj <= 8)
    hipLaunchKernelGGL(qk_norm_rope_kernel<8>, grid, dim3(256), 0, stream, a);
  else if (nj <= 10)
    hipLaunchKernelGGL(qk_norm_rope_kernel<10>, grid, dim3(256), 0, stream, a);
  else if (nj <= 12)
    hipLaunchKernelGGL(qk_norm_rope_kernel<12>, grid, dim3(256), 0, stream, a);
  else if (nj <= 16)
    hipLaunchKernelGGL(qk_norm_rope_kernel<16>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sd
