// Gated fusion O = O_s + g * r * O_lr, r = RMS of the O_s row over d.
//
// robotworld.top SparkDiffusion write-up, section 2.1, the O_i equation (the
// per-token gate starts near zero, so the layer starts near the pure sparse
// branch). D/8 threads own one (batch, token, head) row, 8 channels each;
// the sum of squares is reduced with cross-lane exchanges. Pure streaming:
// reads O_s and O_lr once, writes O once.
#include "sd_device.h"
#include "sd_launch.h"

namespace sd {

__device__ __forceinline__ void load8(const void* base, bool f32, int64_t off, float* v) {
  if (f32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void gate_fuse_kernel(const void* __restrict__ Os, const void* __restrict__ Olr,
                                                        int in_f32, const float* __restrict__ g, int64_t g_sb,
                                                        int64_t g_sl, int64_t g_sh, uint16_t* __restrict__ O, int B,
                                                        int L, int H, int64_t so_b, int64_t so_l, int64_t so_h) {
  constexpr int TPR = D / 8;
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / TPR;
  const int sub = (int)(gt % TPR);
  const int64_t n_rows = (int64_t)B * L * H;
  if (row >= n_rows) return;  // whole TPR-lane groups leave together
  const int h = (int)(row % H);
  const int i = (int)((row / H) % L);
  const int b = (int)(row / ((int64_t)H * L));
  const int64_t off = (int64_t)b * so_b + (int64_t)i * so_l + (int64_t)h * so_h + sub * 8;
  float os[8], lr[8];
  load8(Os, in_f32, off, os);
  load8(Olr, in_f32, off, lr);
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += os[k] * os[k];
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = sqrtf(ss * (1.0f / D));
  const float coef = g[(int64_t)b * g_sb + (int64_t)i * g_sl + (int64_t)h * g_sh] * r;
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(fmaf(coef, lr[2 * k], os[2 * k]), fmaf(coef, lr[2 * k + 1], os[2 * k + 1]));
  *reinterpret_cast<u32x4*>(O + off) = w;
}

hipError_t launch_gate_fuse(const void* Os, const void* Olr, int in_f32, const float* g, int64_t g_sb, int64_t g_sl,
                            int64_t g_sh, void* O, int B, int L, int H, int D, int64_t so_b, int64_t so_l,
                            int64_t so_h, hipStream_t stream) {
  const int64_t threads = (int64_t)B * L * H * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  uint16_t* o = reinterpret_cast<uint16_t*>(O);
  if (D == 128)
    hipLaunchKernelGGL(gate_fuse_kernel<128>, grid, dim3(256), 0, stream, Os, Olr, in_f32, g, g_sb, g_sl, g_sh, o,
                       B, L, H, so_b, so_l, so_h);
  else if (D == 64)
    hipLaunchKernelGGL(gate_fuse_kernel<64>, grid, dim3(256), 0, stream, Os, Olr, in_f32, g, g_sb, g_sl, g_sh, o, B,
                       L, H, so_b, so_l, so_h);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sd
