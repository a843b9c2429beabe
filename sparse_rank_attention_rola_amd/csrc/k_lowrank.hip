// Low-rank compensation branch: RoPE table, the state C = sum_j k~_j v_j^T,
// and its deterministic finalisation.
//
// robotworld.top SparkDiffusion write-up, section 2.1: k~_j = R_r(p_j)
// phi(P_k kn_j) (RoPE applied after the pointwise map phi), C = sum_j
// k~_j v_j^T over all tokens, linear in the sequence length.
//
// lowrank_kv_kernel: one workgroup per (batch, head, run of 64-token tiles).
// Per tile the Kn and V rows are staged through LDS (Kn row-major, V
// transposed); two waves project 32 tokens each onto the rank dims with
// P_k on MFMA, phi is applied and the result parked in a 64 x 33 float LDS
// patch; all threads rotate the RoPE pairs in place; then each wave owns a
// 32-channel slice of C and accumulates k~^T V on MFMA with k~ split into
// bf16 hi + lo parts (V is exact in bf16), so C keeps ~16 significant bits
// per product and f32 accumulation. K and V are read from HBM exactly once.
// Each workgroup writes its partial C; lowrank_finalize_kernel sums the
// partials in a fixed order (bitwise reproducible, no atomics) and emits
// C (f32) and C^T split into bf16 hi/lo for the query side. Under a causal
// window (write-up, section 4) the runs stop at chunk boundaries and each
// chunk's state is the sum of the runs of the chunks it sees.
#include "sd_device.h"
#include "sd_launch.h"
#include "sd_tiles.h"
#include "sd_reduce.h"

namespace sd {

__device__ __forceinline__ float phi_elu1_kv(float x) { return x > 0.f ? x + 1.f : __expf(x); }

__global__ void rope_table_kernel(RopeThetas th, int n, int max_ext, float2* __restrict__ tab) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * max_ext) return;
  const int m = i / max_ext, p = i - m * max_ext;
  double s, c;
  sincos((double)p * (double)th.theta[m], &s, &c);
  tab[i] = make_float2((float)c, (float)s);
}

template <int D>
__global__ __launch_bounds__(256) void lowrank_kv_kernel(LowrankKvArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TileSmem<D>::kElems];
  __shared__ float F[64 * 33];
  const int64_t n_work = (int64_t)a.B * a.H * a.runs.n_runs;
  const int64_t wi = xcd_work_index(blockIdx.x, n_work);
  if (wi < 0) return;
  const int run = (int)(wi % a.runs.n_runs);
  const int64_t bh = wi / a.runs.n_runs;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;

  u32x4 pk[D / 16];
  {
    const uint16_t* P = a.Pk + (int64_t)h * a.P_hs;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      pk[s] = (wv < 2 && l32 < a.rank) ? *reinterpret_cast<const u32x4*>(P + l32 * D + 16 * s + 8 * hf)
                                       : u32x4{0, 0, 0, 0};
  }
  f32x16 cacc = {};
  TileLoader<D, 256> ld;
  const uint16_t* Kb = a.Kn + (int64_t)b * a.sk_b + (int64_t)h * a.sk_h;
  const uint16_t* Vb = a.V + (int64_t)b * a.sv_b + (int64_t)h * a.sv_h;
  int t_begin, t_end, tok_lo, tok_hi;  // tiles of the run, tokens of its chunk
  run_extent(a.runs, a.L, run, t_begin, t_end, tok_lo, tok_hi);
  const int hw = a.Hg * a.Wg;
  for (int tl = t_begin; tl < t_end; ++tl) {
    const int tok0 = tl * 64;
    ld.load(Kb, a.sk_l, Vb, a.sv_l, tok0, a.L, tid);
    __syncthreads();
    ld.store(tile, tid, true);
    __syncthreads();
    if (wv < 2) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        acc = mfma32(as_bf16x8(pk[s]), lds_k_chunk<D>(tile, 32 * wv + l32, 2 * s + hf), acc);
      const int tk = tok0 + 32 * wv + l32;
      const bool tok_ok = tk >= tok_lo && tk < tok_hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ri = 8 * (r >> 2) + 4 * hf + (r & 3);
        F[(32 * wv + l32) * 33 + ri] = (ri < a.rank && tok_ok) ? phi_elu1_kv(acc[r]) : 0.f;
      }
    }
    __syncthreads();
    const int np = a.rope.n;
    for (int it = tid; it < 64 * np; it += 256) {
      const int tk = it / np, m = it - tk * np;
      const int tok = tok0 + tk;
      if (tok < tok_lo || tok >= tok_hi) continue;
      const int axis = a.rope.axis[m];
      const int p = axis == 0 ? tok / hw : (axis == 1 ? (tok / a.Wg) % a.Hg : tok % a.Wg);
      const float2 cs = a.rope_tab[m * a.rope.max_ext + p];
      float* f = F + tk * 33 + a.rope.dim[m];
      const float u = f[0], v = f[1];
      f[0] = u * cs.x - v * cs.y;
      f[1] = u * cs.y + v * cs.x;
    }
    __syncthreads();
    if (wv < D / 32) {
      const uint16_t* Vt = tile + TileSmem<D>::kKElems;
      const int d = 32 * wv + l32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float f8[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) f8[p] = F[(16 * s + 8 * hf + p) * 33 + l32];
        bf16x8 ahi, alo;
        split_bf16x8(f8, ahi, alo);
        const bf16x8 vb = cat_bf16x8(lds_vt_chunk(Vt, d, 4 * s + 2 * hf), lds_vt_chunk(Vt, d, 4 * s + 2 * hf + 1));
        cacc = mfma32(ahi, vb, cacc);
        cacc = mfma32(alo, vb, cacc);
      }
    }
  }
  if (wv < D / 32) {
    float* out = a.partial + ((int64_t)bh * a.runs.n_runs + run) * 32 * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ri = 8 * (r >> 2) + 4 * hf + (r & 3);
      out[ri * D + 32 * wv + l32] = cacc[r];
    }
  }
}

// One thread per (batch*head, chunk, rank slot, channel); the runs of the
// chunk's window are summed in run order (bitwise reproducible).
__global__ void lowrank_finalize_kernel(const float* __restrict__ partial, int64_t BH, RunGeo runs, int n_ar,
                                        int window, int rank, int D, RankRows rows, float* __restrict__ C_out,
                                        uint16_t* __restrict__ Ct_hi, uint16_t* __restrict__ Ct_lo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= BH * n_ar * 32 * D) return;
  const int d = (int)(i % D);
  const int r = (int)((i / D) % 32);
  const int64_t bc = i / (32 * D);  // (batch*head) * n_ar + chunk
  const int c = (int)(bc % n_ar);
  const int64_t bh = bc / n_ar;
  const int row = rows.row[r];
  float s = 0.f;
  if (row >= 0) {
    const int c0 = window > 0 ? max(0, c - window + 1) : 0;
    const float* p = partial + (bh * runs.n_runs * 32 + row) * D + d;
    s = strided_sum_in_order(p, 32 * D, c0 * runs.runs_per_ar, (c + 1) * runs.runs_per_ar);
  }
  if (C_out && r < rank) C_out[(bc * rank + r) * D + d] = s;
  const __bf16 hi = (__bf16)s;
  const __bf16 lo = (__bf16)(s - (float)hi);
  Ct_hi[(bc * D + d) * 32 + r] = __builtin_bit_cast(uint16_t, hi);
  Ct_lo[(bc * D + d) * 32 + r] = __builtin_bit_cast(uint16_t, lo);
}

hipError_t launch_rope_table(const RopeThetas& th, int n, int max_ext, float2* tab, hipStream_t stream) {
  const int total = n * max_ext;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, th, n, max_ext, tab);
  return hipGetLastError();
}

hipError_t launch_lowrank_kv(const LowrankKvArgs& a, int D, hipStream_t stream) {
  const int64_t n_work = (int64_t)a.B * a.H * a.runs.n_runs;
  const int64_t grid = (n_work + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (D == 128)
    hipLaunchKernelGGL(lowrank_kv_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL(lowrank_kv_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lowrank_finalize(const float* partial, int BH, const RunGeo& runs, int n_ar, int window, int rank,
                                   int D, const RankRows& rows, float* C_out, uint16_t* Ct_hi, uint16_t* Ct_lo,
                                   hipStream_t stream) {
  const int64_t total = (int64_t)BH * n_ar * 32 * D;
  hipLaunchKernelGGL(lowrank_finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, partial,
                     (int64_t)BH, runs, n_ar, window, rank, D, rows, C_out, Ct_hi, Ct_lo);
  return hipGetLastError();
}

}  // namespace sd
