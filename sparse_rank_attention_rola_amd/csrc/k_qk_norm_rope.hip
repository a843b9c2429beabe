// Fused q/k producer of the attention block: RMSNorm of each token's
// projection row, then the backbone 3D RoPE on every head (robotworld.top
// SparkDiffusion write-up, section 2.1: the low-rank branch reuses the
// normalised q/k from before the backbone attention; kais-engine portability
// report, section 2.1: fused QKV + RoPE operator).
//
//   y_c  = x_c / sqrt(mean_c' x_c'^2 + eps) * gamma_c      (Qn / Kn, bf16)
//   out  = R(p) y per head, pairs (2m, 2m+1) rotated       (Q / K, bf16)
//
// One wavefront streams one row (a token's q or k, H*d channels): lane l
// holds 16-byte chunks l, l + 64, ... of the row, all at the same offset
// inside a head (64 is a multiple of the d/8 chunks of a head), so every
// lane rotates the same 4 channel pairs at every head and computes their
// cos/sin once per row. The workgroups are persistent: a wave handles rows
// of one tensor only and keeps that tensor's gamma in registers.
#include "sd_device.h"
#include "sd_launch.h"

namespace sd {

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
