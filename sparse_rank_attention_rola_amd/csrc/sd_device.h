// Device-side helpers shared by the libsd kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

// MFMA operand and accumulator registers.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 floats -> MFMA bf16 operand (nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
  return r;
}

// Split 8 floats into bf16 hi + bf16 lo parts (x ~= hi + lo to ~16 bits).
__device__ __forceinline__ void split_bf16x8(const float* f, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __bf16 h = (__bf16)f[i];
    hi[i] = h;
    lo[i] = (__bf16)(f[i] - (float)h);
  }
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup id remap so that consecutive work items land on the same XCD:
// the hardware deals workgroups to the 8 XCDs round-robin, so workgroup i
// runs on XCD i % 8. Returns the work index, or -1 for padding workgroups.
// The grid must have round_up(n_work, 8) workgroups.
__device__ __forceinline__ int64_t xcd_work_index(int64_t wg, int64_t n_work) {
  const int64_t per = (n_work + kNumXcd - 1) / kNumXcd;
  const int64_t w = (wg % kNumXcd) * per + wg / kNumXcd;
  return w < n_work ? w : -1;
}

// Workgroup -> (group, item) map that keeps all XCDs on the same group at a
// time: group g (a batch-head) is split into 8 contiguous runs of items (query
// blocks), run x going to XCD x. Concurrent workgroups then share one head's
// K/V in the last-level cache while each XCD's L2 sees a contiguous run.
// The grid must have 8 * ceil(items / 8) * groups workgroups; returns false
// for padding workgroups.
__device__ __forceinline__ bool xcd_group_item(int64_t wg, int items, int64_t groups, int64_t& group, int& item) {
  const int per = (items + kNumXcd - 1) / kNumXcd;
  const int64_t j = wg / kNumXcd;
  group = j / per;
  item = (int)(wg % kNumXcd) * per + (int)(j % per);
  return group < groups && item < items;
}

// Value of lane l ^ 32 (v_permlane32_swap: one VALU op, no LDS traffic).
__device__ __forceinline__ float partner32(float x, int hf) {
  const int xi = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float(hf ? r[0] : r[1]);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef int int2v __attribute__((ext_vector_type(2)));

// Lane-exchange helpers for float64 values (two 32-bit moves each, VALU only).
template <int CTRL>  // DPP control, e.g. 0x120 + n = rotate right by n within a row of 16
__device__ __forceinline__ double dpp_f64(double v) {
  const int2v p = __builtin_bit_cast(int2v, v);
  int2v r;
  r[0] = __builtin_amdgcn_update_dpp(0, p[0], CTRL, 0xF, 0xF, false);
  r[1] = __builtin_amdgcn_update_dpp(0, p[1], CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, r);
}

// value of lane l ^ 16 (v_permlane16_swap exchanges the odd and even rows)
__device__ __forceinline__ double partner16_f64(double v, int lane) {
  const int2v p = __builtin_bit_cast(int2v, v);
  const auto a = __builtin_amdgcn_permlane16_swap(p[0], p[0], false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(p[1], p[1], false, false);
  const bool odd = (lane >> 4) & 1;
  int2v r;
  r[0] = odd ? a[0] : a[1];
  r[1] = odd ? b[0] : b[1];
  return __builtin_bit_cast(double, r);
}

__device__ __forceinline__ double partner32_f64(double v, int lane) {
  const int2v p = __builtin_bit_cast(int2v, v);
  const auto a = __builtin_amdgcn_permlane32_swap(p[0], p[0], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(p[1], p[1], false, false);
  const bool up = lane >= 32;
  int2v r;
  r[0] = up ? a[0] : a[1];
  r[1] = up ? b[0] : b[1];
  return __builtin_bit_cast(double, r);
}

// Sum of v over the lanes of a wave that agree on lane % G (G = 2 or 4), in a
// fixed order; every lane receives its class's sum.
template <int G>
__device__ __forceinline__ double sum_lanes_mod(double v, int lane) {
  if constexpr (G == 2) v += dpp_f64<0x122>(v);
  v += dpp_f64<0x124>(v);
  v += dpp_f64<0x128>(v);
  v += partner16_f64(v, lane);
  v += partner32_f64(v, lane);
  return v;
}

// Sum of the 8 bf16 values of an MFMA operand, accumulated into acc (f32).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace sd
