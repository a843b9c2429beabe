// Backward of the RoLA attention layer (block map held fixed).
//
// SparkDiffusion README_zh (distillation and operators sections): training
// the sparse student needs a backward kernel of its sparse + low-rank
// attention, whose forward is the robotworld.top write-up, section 2.1:
//   O_i = O_s,i + g_i r_i O_lr,i,  O_lr,i = w * y_i / rho_i,  y_i = C^T q~_i,
//   C = sum_j k~_j v_j^T,  q~ = R phi(P_q qn),  k~ = R phi(P_k kn).
// The gradients are the exact derivatives of that forward (chain rule):
//   dg_i = r_i (dO_i . O_lr,i),  dO_s,i = dO_i + g_i (dO_i . O_lr,i) O_s,i / (d r_i),
//   dy_i = u_i / rho_i - y_i (u_i . y_i) / (d rho_i^3),  u_i = w * g_i r_i dO_i,
//   dq~_i = C dy_i,  dC = sum_i q~_i dy_i^T,  dk~_j = dC v_j,  dv_j += dC^T k~_j,
//   then back through R (rotation by the negative angle), phi' and the
//   projections; and the softmax branch as in attention backward:
//   D_i = dO_s,i . O_s,i, dS = P * (dO_s V^T - D), dQ = scale dS K,
//   dK = scale dS^T Q, dV += P^T dO_s.
// Under a causal window every chunk has its own state: the query side uses
// the state of its chunk, and a key receives the sum of dC over the chunks
// that see it.
//
// Kernels:
//   bwd_query_kernel    per 32 queries (one wave): recompute q~ and y, the
//                       gate / RMS / RMSNorm derivatives, dq~ = C dy on
//                       MFMA, back through RoPE and phi, dQn = P_q^T da;
//                       writes dO_s (bf16), D, q~, dy, da and dg per head.
//   token_outer_kernel  sum over a run of tokens of X^T Y (X: 32 columns)
//                       on MFMA with hi/lo bf16 operands: the partial dC
//                       (q~, dy) and dP_q / dP_k (da / db, qn / kn).
//   dstate_finalize / dproj_finalize: fixed-order sums of the partials.
//   bwd_key_kernel      per 32 keys: recompute k~, dk~ = dC v, dv += dC^T k~,
//                       back through RoPE and phi, dKn = P_k^T db.
//   transpose_map_kernel  per (batch, head): the query blocks that keep
//                       each key block, ascending (a counting sort).
//   bwd_dq_kernel       per query block, like the forward loop: S^T, P^T
//                       from the saved log-sum-exp, dP^T = V dO_s^T, dS^T,
//                       dQ^T += K^T dS^T (K^T by transposing LDS reads; the
//                       K tile is read both ways, so it is kept with the
//                       u_swz chunk swizzle that serves both without bank
//                       conflicts).
//   bwd_dkdv_kernel     per key block (K, V staged in LDS once), over the
//                       query blocks that keep it: S = Q K^T, dP = dO_s V^T,
//                       dV^T += dO_s^T P and dK^T += Q^T dS (transposing
//                       reads of the staged Q and dO_s tiles); each head's
//                       key blocks launched longest query list first.
// Every sum runs in a fixed order: the results are bitwise reproducible.
#include "sd_device.h"
#include "sd_launch.h"
#include "sd_tiles.h"
#include "sd_reduce.h"

namespace sd {

__device__ __forceinline__ float phi_b(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ float dphi_b(float x) { return x > 0.f ? 1.f : __expf(x); }

// Channel of accumulator register r of an O^T tile dt (lane half hf).
__device__ __forceinline__ int och(int dt, int r, int hf) { return 32 * dt + 8 * (r >> 2) + 4 * hf + (r & 3); }

// The 8 channels 16 s + 8 hf .. +7 of the lane's token (the MFMA B-operand
// slice) from values held in the O^T accumulator layout: each lane holds 4
// of every 8 channels; one lane-pair exchange per value completes the slice.
template <int D>
__device__ __forceinline__ void otile_slice(const f32x16 (&v)[D / 32], int s, int hf, float out[8]) {
  const int g0 = 2 * s, g1 = 2 * s + 1;
  float own0[4], own1[4], y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    own0[e] = v[g0 >> 2][4 * (g0 & 3) + e];
    own1[e] = v[g1 >> 2][4 * (g1 & 3) + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = partner32(hf ? own0[e] : own1[e], hf);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = hf ? y[e] : own0[e];
    out[4 + e] = hf ? own1[e] : y[e];
  }
}

__device__ __forceinline__ void load8_split(const float* p, bool ok, bf16x8& hi, bf16x8& lo) {
  float f[8];
  if (ok) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
    const f32x4 w = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = u[e];
      f[4 + e] = w[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0.f;
  }
  split_bf16x8(f, hi, lo);
}

// The cos/sin of the RoPE pairs a lane rotates in a wave's 32 x 33 patch
// (lane l32 = token tok0 + l32; the two lane halves take alternate pairs),
// loaded once at the start of a kernel so that their latency overlaps its
// other loads; both rotations use them. With kConst the pair arguments are
// read at constant indices and picked by lane half (no memory load and wait
// for a lane-indexed argument read); the query side measured faster that
// way, the key side slower, so each takes its own.
struct RopeLane {
  float2 cs[kMaxRopePairs / 2];
};

template <bool kConst>
__device__ __forceinline__ void rope_lane_load(RopeLane& rl, const float2* tab, const RopeArgs& rope, int Hg, int Wg,
                                               int tok0, int lane) {
  const int hf = lane >> 5, l32 = lane & 31;
  const int tok = tok0 + l32;
  const int hw = Hg * Wg;
  const int pos[3] = {min(tok / hw, rope.max_ext - 1), (tok / Wg) % Hg, tok % Wg};
#pragma unroll
  for (int j = 0; j < kMaxRopePairs / 2; ++j) {
    const int m = 2 * j + hf;
    rl.cs[j] = float2{1.f, 0.f};
    if (2 * j < rope.n && m < rope.n) {
      const int axis = kConst ? (hf ? rope.axis[2 * j + 1] : rope.axis[2 * j]) : rope.axis[m];
      rl.cs[j] = tab[m * rope.max_ext + (axis == 0 ? pos[0] : axis == 1 ? pos[1] : pos[2])];
    }
  }
}

// Rotates the RoPE pairs of the patch by +angle (dir = 1) or by -angle
// (dir = -1, the transpose).
template <bool kConst>
__device__ __forceinline__ void rope_patch(float* F, const RopeLane& rl, const RopeArgs& rope, int lane, int dir) {
  const int hf = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int j = 0; j < kMaxRopePairs / 2; ++j) {
    const int m = 2 * j + hf;
    if (2 * j < rope.n && m < rope.n) {
      const float2 cs = rl.cs[j];
      const float sn = dir > 0 ? cs.y : -cs.y;
      float* f = F + l32 * 33 + (kConst ? (hf ? rope.dim[2 * j + 1] : rope.dim[2 * j]) : rope.dim[m]);
      const float u = f[0], v = f[1];
      f[0] = u * cs.x - v * sn;
      f[1] = u * sn + v * cs.x;
    }
  }
}

// ---------------------------------------------------------------------------
// Query side of the low-rank branch, gate and RMS coupling.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_query_kernel(BwdArgs a) {
  __shared__ float Fw[4][32 * 33];
  __shared__ float Fa[4][32 * 33];
  int64_t bh;
  int blk;
  if (!xcd_group_item(blockIdx.x, (a.L + 127) / 128, (int64_t)a.B * a.H, bh, blk)) return;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int tok0 = blk * 128 + 32 * wv;
  const int q_tok = tok0 + l32;
  const bool q_ok = q_tok < a.L;
  const int q_cl = min(q_tok, a.L - 1);
  const int q_chunk = q_cl / a.ar_tokens;
  const int n_ar = (a.L + a.ar_tokens - 1) / a.ar_tokens;
  const int c_first = __builtin_amdgcn_readfirstlane(q_chunk);
  const int c_last = __builtin_amdgcn_readlane(q_chunk, 31);
  float* fw = Fw[wv];
  float* fa = Fa[wv];
  const int64_t row = ((int64_t)b * a.L + q_cl) * a.H + h;
  RopeLane rl;
  rope_lane_load<true>(rl, a.rope_tab, a.rope, a.Hg, a.Wg, tok0, lane);
  const float rr = q_ok ? a.rms[row] : 0.f;
  const float gv = q_ok ? a.g[(int64_t)b * a.g_sb + (int64_t)q_cl * a.g_sl + (int64_t)h * a.g_sh] : 0.f;

  // 1. a = P_q qn (pre-phi in Fa), q~ = R phi(a) (in Fw)
  {
    u32x4 qreg[D / 16];
    const uint16_t* qp = a.Qn + (int64_t)b * a.sq_b + (int64_t)q_cl * a.sq_l + (int64_t)h * a.sq_h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qreg[s] = q_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
    const uint16_t* Pq = a.Pq + (int64_t)h * a.P_hs;
    // all of P_q's operands are loaded before the products (one wait on
    // memory, not one per product; the fence keeps them apart)
    u32x4 pqa[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      pqa[s] = (l32 < a.rank) ? *reinterpret_cast<const u32x4*>(Pq + l32 * D + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc = mfma32(as_bf16x8(pqa[s]), as_bf16x8(qreg[s]), acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ri = 8 * (r >> 2) + 4 * hf + (r & 3);
      fa[l32 * 33 + ri] = ri < a.rank ? acc[r] : 0.f;
      fw[l32 * 33 + ri] = ri < a.rank ? phi_b(acc[r]) : 0.f;
    }
  }
  __syncthreads();
  rope_patch<true>(fw, rl, a.rope, lane, 1);
  __syncthreads();
  bf16x8 qhi[2], qlo[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float t8[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) t8[p] = fw[l32 * 33 + 16 * s + 8 * hf + p];
    split_bf16x8(t8, qhi[s], qlo[s]);
    if (q_ok) {
      float* dst = a.qt + row * 32 + 16 * s + 8 * hf;
      *reinterpret_cast<f32x4*>(dst) = f32x4{t8[0], t8[1], t8[2], t8[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{t8[4], t8[5], t8[6], t8[7]};
    }
  }

  // 2. y = C^T q~ with the state of the lane's chunk (each chunk's state
  // loaded whole before its products)
  f32x16 yv[D / 32];
  for (int c = c_first; c <= c_last; ++c) {
    const int64_t cbase = (bh * n_ar + c) * D * 32;
    const bool mine = q_chunk == c;
    // one channel tile of the state at a time, the next one loading while
    // the current one is used
    u32x4 cth[2][2], ctl[2][2];
    auto load_ct = [&](int dt, u32x4 (&th)[2], u32x4 (&tl)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t off = cbase + (int64_t)(32 * dt + l32) * 32 + 16 * s + 8 * hf;
        th[s] = *reinterpret_cast<const u32x4*>(a.Ct_hi + off);
        tl[s] = *reinterpret_cast<const u32x4*>(a.Ct_lo + off);
      }
    };
    load_ct(0, cth[0], ctl[0]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      if (dt + 1 < D / 32) load_ct(dt + 1, cth[(dt + 1) & 1], ctl[(dt + 1) & 1]);
      f32x16 y = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ch = as_bf16x8(cth[dt & 1][s]);
        const bf16x8 cl = as_bf16x8(ctl[dt & 1][s]);
        y = mfma32(ch, qhi[s], y);
        y = mfma32(cl, qhi[s], y);
        y = mfma32(ch, qlo[s], y);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) yv[dt][r] = (c == c_first || mine) ? y[r] : yv[dt][r];
    }
  }

  // 3. RMSNorm, gate and RMS coupling, per query (lane pair); dO and O_s
  // (their 4-channel groups in the accumulator layout) are loaded here
  const uint16_t* dop = a.dO + (int64_t)b * a.so_b + (int64_t)q_cl * a.so_l + (int64_t)h * a.so_h;
  const uint16_t* osp = a.Os + row * D;
  u32x2 do2[D / 32][4], os2[D / 32][4], w2[D / 32][4];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int c0 = och(dt, 4 * rg, hf);
      do2[dt][rg] = q_ok ? *reinterpret_cast<const u32x2*>(dop + c0) : u32x2{0, 0};
      os2[dt][rg] = q_ok ? *reinterpret_cast<const u32x2*>(osp + c0) : u32x2{0, 0};
      w2[dt][rg] = a.rmsw ? *reinterpret_cast<const u32x2*>(a.rmsw + c0) : u32x2{0x3F803F80u, 0x3F803F80u};
    }
  // the packed values are opaque to the compiler between the loops below, so
  // each loop unpacks them again instead of keeping 64 unpacked floats live
  auto reopen = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        asm volatile("" : "+v"(do2[dt][rg]));
        asm volatile("" : "+v"(w2[dt][rg]));
      }
  };
  float ss = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss += yv[dt][r] * yv[dt][r];
  ss += partner32(ss, hf);
  const float inv = rsqrtf(ss * (1.0f / D) + a.eps);
  // dO and O_s stay packed (bf16 pairs) and are unpacked where used, so
  // that no f32 copy of them is live beside y
  auto unpack = [&](const u32x2& v2, int e) __attribute__((always_inline)) {
    return (e & 1) ? bf16_hi(v2[e >> 1]) : bf16_lo(v2[e >> 1]);
  };
  float t = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int c0 = och(dt, 4 * rg, hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rg + e;
        t += unpack(do2[dt][rg], e) * unpack(w2[dt][rg], e) * yv[dt][r] * inv;
      }
    }
  t += partner32(t, hf);
  if (q_ok && hf == 0) a.dg_head[row] = rr * t;
  const float coef = rr > 0.f ? gv * t / ((float)D * rr) : 0.f;
  const float gr = gv * rr;
  float dsum = 0.f, uy = 0.f;
  reopen();
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int c0 = och(dt, 4 * rg, hf);
      float dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rg + e;
        const float dov = unpack(do2[dt][rg], e), osv = unpack(os2[dt][rg], e);
        const float v = fmaf(coef, osv, dov);
        dsv[e] = bf16_bits_to_f32(f32_to_bf16_bits(v));
        dsum += dsv[e] * osv;
        uy += unpack(w2[dt][rg], e) * gr * dov * yv[dt][r];  // u y
      }
      if (q_ok) {
        u32x2 o;
        o[0] = pack_bf16x2(dsv[0], dsv[1]);
        o[1] = pack_bf16x2(dsv[2], dsv[3]);
        *reinterpret_cast<u32x2*>(a.dOs + row * D + c0) = o;
      }
    }
  dsum += partner32(dsum, hf);
  uy += partner32(uy, hf);
  if (q_ok && hf == 0) a.Dd[bh * a.L + q_cl] = dsum;
  const float k3 = uy * inv * inv * inv * (1.0f / D);
  reopen();
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rg + e;
        const float u = unpack(w2[dt][rg], e) * gr * unpack(do2[dt][rg], e);
        yv[dt][r] = u * inv - yv[dt][r] * k3;  // dy
      }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      if (q_ok)
        *reinterpret_cast<f32x4*>(a.dy + row * D + och(dt, 4 * rg, hf)) =
            f32x4{yv[dt][4 * rg], yv[dt][4 * rg + 1], yv[dt][4 * rg + 2], yv[dt][4 * rg + 3]};
  }

  // 4. dq~ = C dy (rank x token), the state of the lane's chunk
  bf16x8 dyh[D / 16], dyl[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    float f8[8];
    otile_slice<D>(yv, s, hf, f8);
    split_bf16x8(f8, dyh[s], dyl[s]);
  }
  f32x16 dq = {};
  for (int c = c_first; c <= c_last; ++c) {
    const float* Cr = a.C + (bh * n_ar + c) * (int64_t)a.rank * D;
    const bool mine = q_chunk == c;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 chi, clo;
      load8_split(Cr + (int64_t)l32 * D + 16 * s + 8 * hf, l32 < a.rank, chi, clo);
      acc = mfma32(chi, dyh[s], acc);
      acc = mfma32(clo, dyh[s], acc);
      acc = mfma32(chi, dyl[s], acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[r] = (c == c_first || mine) ? acc[r] : dq[r];
  }

  // 5. da = R^T dq~ * phi'(a); the rotation is read again here rather than
  // held in registers through phases 2-4 (from opaque copies of the lane and
  // grid sizes, so that the compiler does not keep the first call's
  // divisions and masks instead)
  int lane5 = lane, hg = a.Hg, wg = a.Wg;
  asm volatile("" : "+v"(lane5), "+s"(hg), "+s"(wg));
  rope_lane_load<true>(rl, a.rope_tab, a.rope, hg, wg, tok0, lane5);
  __syncthreads();  // every wave is done reading q~ from its patch
#pragma unroll
  for (int r = 0; r < 16; ++r) fw[l32 * 33 + 8 * (r >> 2) + 4 * hf + (r & 3)] = dq[r];
  __syncthreads();
  rope_patch<true>(fw, rl, a.rope, lane5, -1);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = l32 * 33 + 8 * (r >> 2) + 4 * hf + (r & 3);
    fw[i] *= dphi_b(fa[i]);
  }
  __syncthreads();
  bf16x8 dah[2], dal[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float t8[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) t8[p] = fw[l32 * 33 + 16 * s + 8 * hf + p];
    split_bf16x8(t8, dah[s], dal[s]);
    if (q_ok) {
      float* dst = a.da + row * 32 + 16 * s + 8 * hf;
      *reinterpret_cast<f32x4*>(dst) = f32x4{t8[0], t8[1], t8[2], t8[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{t8[4], t8[5], t8[6], t8[7]};
    }
  }

  // 6. dqn = P_q^T da (channel x token)
  const uint16_t* Pq = a.Pq + (int64_t)h * a.P_hs;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rk = 16 * s + 8 * hf + e;
        pa[e] = __builtin_bit_cast(__bf16, rk < a.rank ? Pq[rk * D + 32 * dt + l32] : (uint16_t)0);
      }
      acc = mfma32(pa, dah[s], acc);
      acc = mfma32(pa, dal[s], acc);
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      if (q_ok)
        *reinterpret_cast<f32x4*>(a.dQn + row * D + och(dt, 4 * rg, hf)) =
            f32x4{acc[4 * rg], acc[4 * rg + 1], acc[4 * rg + 2], acc[4 * rg + 3]};
  }
}

// ---------------------------------------------------------------------------
// Sums over runs of tokens of X^T Y.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void token_outer_kernel(const float* __restrict__ X, const float* __restrict__ Yf,
                                                          const uint16_t* __restrict__ Yb, int64_t y_sb, int64_t y_sl,
                                                          int64_t y_sh, int B, int H, int L, RunGeo runs,
                                                          float* __restrict__ part) {
  __shared__ float Xs[64][33];
  __shared__ float Ys[64][D + 1];
  const int64_t nbh = (int64_t)B * H;
  const int64_t bh = blockIdx.x % nbh;
  const int run = (int)(blockIdx.x / nbh);
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  int t_begin, t_end, lo, hi;
  run_extent(runs, L, run, t_begin, t_end, lo, hi);
  f32x16 acc = {};
  for (int tl = t_begin; tl < t_end; ++tl) {
    const int tok0 = tl * 64;
    __syncthreads();
    // X tile: 64 tokens x 32 (8 floats per thread); Y tile: 64 x D
    {
      const int t = tid >> 2, c = (tid & 3) * 8;
      const int tok = tok0 + t;
      const bool ok = tok >= lo && tok < hi;
      const float* xp = X + (((int64_t)b * L + tok) * H + h) * 32 + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) Xs[t][c + e] = ok ? xp[e] : 0.f;
    }
    for (int i = tid; i < 64 * (D / 8); i += 256) {
      const int t = i / (D / 8), c = (i % (D / 8)) * 8;
      const int tok = tok0 + t;
      const bool ok = tok >= lo && tok < hi;
      if (Yf) {
        const float* yp = Yf + (((int64_t)b * L + tok) * H + h) * D + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) Ys[t][c + e] = ok ? yp[e] : 0.f;
      } else {
        const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(Yb + (int64_t)b * y_sb + (int64_t)tok * y_sl +
                                                              (int64_t)h * y_sh + c)
                           : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Ys[t][c + 2 * e] = bf16_lo(v[e]);
          Ys[t][c + 2 * e + 1] = bf16_hi(v[e]);
        }
      }
    }
    __syncthreads();
    if (wv < D / 32) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float xa[8], yb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xa[e] = Xs[16 * st + 8 * hf + e][l32];
          yb[e] = Ys[16 * st + 8 * hf + e][32 * wv + l32];
        }
        bf16x8 xh, xl, yh, yl;
        split_bf16x8(xa, xh, xl);
        split_bf16x8(yb, yh, yl);
        acc = mfma32(xh, yh, acc);
        acc = mfma32(xl, yh, acc);
        acc = mfma32(xh, yl, acc);
      }
    }
  }
  if (wv < D / 32) {
    float* out = part + ((int64_t)bh * runs.n_runs + run) * 32 * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(8 * (r >> 2) + 4 * hf + (r & 3)) * D + 32 * wv + l32] = acc[r];
  }
}

// dC seen by chunk c: runs of chunks c .. last, in run order.
__global__ void dstate_finalize_kernel(const float* __restrict__ part, int64_t BH, RunGeo runs, int n_ar, int window,
                                       int D, float* __restrict__ dC, uint16_t* __restrict__ dCt_hi,
                                       uint16_t* __restrict__ dCt_lo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= BH * n_ar * 32 * D) return;
  const int d = (int)(i % D);
  const int r = (int)((i / D) % 32);
  const int64_t bc = i / (32 * D);
  const int c = (int)(bc % n_ar);
  const int64_t bh = bc / n_ar;
  const int last = window > 0 ? min(n_ar - 1, c + window - 1) : n_ar - 1;
  const float* p = part + (bh * runs.n_runs * 32 + r) * D + d;
  const float s = strided_sum_in_order(p, 32 * D, c * runs.runs_per_ar, (last + 1) * runs.runs_per_ar);
  dC[(bc * 32 + r) * D + d] = s;
  const __bf16 hi = (__bf16)s;
  const __bf16 lo = (__bf16)(s - (float)hi);
  dCt_hi[(bc * D + d) * 32 + r] = __builtin_bit_cast(uint16_t, hi);
  dCt_lo[(bc * D + d) * 32 + r] = __builtin_bit_cast(uint16_t, lo);
}

// 64 output elements per workgroup; its 4 waves sum contiguous quarters of
// the partial list (b, h, run order) with coalesced loads, then the quarters
// are added in order.
__global__ __launch_bounds__(256) void dproj_finalize_kernel(const float* __restrict__ part, int B, int H, int n_runs,
                                                             int rank, int D, int per_head, float* __restrict__ dP) {
  __shared__ float q4[4][64];
  const int n_out = per_head ? H : 1;
  const int64_t total = (int64_t)n_out * rank * D;
  const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int qt = threadIdx.x >> 6;
  float s = 0.f;
  if (i < total) {
    const int d = (int)(i % D);
    const int r = (int)((i / D) % rank);
    const int o = (int)(i / ((int64_t)rank * D));
    const int hs = per_head ? 1 : H;  // heads per output
    const int64_t n = (int64_t)B * hs * n_runs;
    const int64_t u0 = n * qt / 4, u1 = n * (qt + 1) / 4;
    // partial u = (b, head hh of the output's heads, run), run fastest;
    // walked in order with incremented indices (no division per term)
    int run = (int)(u0 % n_runs);
    const int64_t bh0 = u0 / n_runs;
    int hh = (int)(bh0 % hs), b = (int)(bh0 / hs);
    const float* pr = part + (int64_t)r * D + d;
    // 8 terms loaded before they are added (in the same order), so that 8
    // loads are in flight instead of one
    for (int64_t u = u0; u < u1; u += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = 0.f;
        if (u + j < u1) {
          const int h = per_head ? o : hh;
          v[j] = pr[(((int64_t)b * H + h) * n_runs + run) * 32 * D];
          if (++run == n_runs) {
            run = 0;
            if (++hh == hs) {
              hh = 0;
              ++b;
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (u + j < u1) s += v[j];
    }
  }
  q4[qt][threadIdx.x & 63] = s;
  __syncthreads();
  if (qt == 0 && i < total) dP[i] = ((q4[0][threadIdx.x] + q4[1][threadIdx.x]) + q4[2][threadIdx.x]) + q4[3][threadIdx.x];
}

// The gate gradient at the gate's own strides. A stride of 0 means the gate
// is broadcast over that dimension (one gate per token for every head, a
// gate shared by the batch, ...): the stored element then receives the sum
// over every (b, l, h) that reads it. One thread per stored element, summing
// in a fixed order (b, then l, then h), so the result is deterministic.
__global__ void dgate_kernel(const float* __restrict__ dg_head, int B, int L, int H, int64_t g_sb, int64_t g_sl,
                             int64_t g_sh, float* __restrict__ dg) {
  const int Bo = g_sb ? B : 1, Lo = g_sl ? L : 1, Ho = g_sh ? H : 1;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)Bo * Lo * Ho) return;
  const int ho = (int)(i % Ho);
  const int64_t r = i / Ho;
  const int lo = (int)(r % Lo), bo = (int)(r / Lo);
  const int b0 = Bo == 1 ? 0 : bo, b1 = Bo == 1 ? B : bo + 1;
  const int l0 = Lo == 1 ? 0 : lo, l1 = Lo == 1 ? L : lo + 1;
  const int h0 = Ho == 1 ? 0 : ho, h1 = Ho == 1 ? H : ho + 1;
  float s = 0.f;
  for (int b = b0; b < b1; ++b)
    for (int l = l0; l < l1; ++l)
      for (int h = h0; h < h1; ++h) s += dg_head[((int64_t)b * L + l) * H + h];
  dg[(int64_t)bo * g_sb + (int64_t)lo * g_sl + (int64_t)ho * g_sh] = s;
}

// ---------------------------------------------------------------------------
// Key side of the low-rank branch.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_key_kernel(BwdArgs a) {
  __shared__ float Fw[4][32 * 33];
  __shared__ float Fa[4][32 * 33];
  int64_t bh;
  int blk;
  if (!xcd_group_item(blockIdx.x, (a.L + 127) / 128, (int64_t)a.B * a.H, bh, blk)) return;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int tok0 = blk * 128 + 32 * wv;
  const int k_tok = tok0 + l32;
  const bool k_ok = k_tok < a.L;
  const int k_cl = min(k_tok, a.L - 1);
  const int k_chunk = k_cl / a.ar_tokens;
  const int n_ar = (a.L + a.ar_tokens - 1) / a.ar_tokens;
  const int c_first = __builtin_amdgcn_readfirstlane(k_chunk);
  const int c_last = __builtin_amdgcn_readlane(k_chunk, 31);
  float* fw = Fw[wv];
  float* fa = Fa[wv];
  const int64_t row = ((int64_t)b * a.L + k_cl) * a.H + h;
  RopeLane rl;
  rope_lane_load<false>(rl, a.rope_tab, a.rope, a.Hg, a.Wg, tok0, lane);

  // 1. b = P_k kn (pre-phi in Fa), k~ = R phi(b) (in Fw)
  {
    u32x4 kreg[D / 16];
    const uint16_t* kp = a.Kn + (int64_t)b * a.sk_b + (int64_t)k_cl * a.sk_l + (int64_t)h * a.sk_h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      kreg[s] = k_ok ? *reinterpret_cast<const u32x4*>(kp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
    const uint16_t* Pk = a.Pk + (int64_t)h * a.P_hs;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 pa = (l32 < a.rank) ? *reinterpret_cast<const u32x4*>(Pk + l32 * D + 16 * s + 8 * hf)
                                      : u32x4{0, 0, 0, 0};
      acc = mfma32(as_bf16x8(pa), as_bf16x8(kreg[s]), acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ri = 8 * (r >> 2) + 4 * hf + (r & 3);
      fa[l32 * 33 + ri] = ri < a.rank ? acc[r] : 0.f;
      fw[l32 * 33 + ri] = ri < a.rank ? phi_b(acc[r]) : 0.f;
    }
  }
  __syncthreads();
  rope_patch<false>(fw, rl, a.rope, lane, 1);
  __syncthreads();
  bf16x8 khi[2], klo[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float t8[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) t8[p] = fw[l32 * 33 + 16 * s + 8 * hf + p];
    split_bf16x8(t8, khi[s], klo[s]);
  }
  u32x4 vreg[D / 16];
  {
    const uint16_t* vp = a.V + (int64_t)b * a.sv_b + (int64_t)k_cl * a.sv_l + (int64_t)h * a.sv_h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      vreg[s] = k_ok ? *reinterpret_cast<const u32x4*>(vp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
  }

  // 2. dk~ = dC v (rank x key) and dv = dC^T k~ (channel x key), with the
  // state gradient seen by the lane's chunk
  f32x16 dk = {};
  f32x16 dv[D / 32];
  for (int c = c_first; c <= c_last; ++c) {
    const int64_t bc = bh * n_ar + c;
    const bool mine = k_chunk == c;
    const bool take = c == c_first || mine;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 chi, clo;
      load8_split(a.dC + (bc * 32 + l32) * D + 16 * s + 8 * hf, true, chi, clo);
      acc = mfma32(chi, as_bf16x8(vreg[s]), acc);
      acc = mfma32(clo, as_bf16x8(vreg[s]), acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[r] = take ? acc[r] : dk[r];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      f32x16 y = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t off = (bc * D + 32 * dt + l32) * 32 + 16 * s + 8 * hf;
        const bf16x8 ch = as_bf16x8(*reinterpret_cast<const u32x4*>(a.dCt_hi + off));
        const bf16x8 cl = as_bf16x8(*reinterpret_cast<const u32x4*>(a.dCt_lo + off));
        y = mfma32(ch, khi[s], y);
        y = mfma32(cl, khi[s], y);
        y = mfma32(ch, klo[s], y);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dv[dt][r] = take ? y[r] : dv[dt][r];
    }
  }
  if (k_ok) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float* p = a.dV + row * D + och(dt, 4 * rg, hf);
        f32x4 v = *reinterpret_cast<f32x4*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += dv[dt][4 * rg + e];
        *reinterpret_cast<f32x4*>(p) = v;
      }
  }

  // 3. db = R^T dk~ * phi'(b)
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) fw[l32 * 33 + 8 * (r >> 2) + 4 * hf + (r & 3)] = dk[r];
  __syncthreads();
  rope_patch<false>(fw, rl, a.rope, lane, -1);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = l32 * 33 + 8 * (r >> 2) + 4 * hf + (r & 3);
    fw[i] *= dphi_b(fa[i]);
  }
  __syncthreads();
  bf16x8 dbh[2], dbl[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float t8[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) t8[p] = fw[l32 * 33 + 16 * s + 8 * hf + p];
    split_bf16x8(t8, dbh[s], dbl[s]);
    if (k_ok) {
      float* dst = a.db + row * 32 + 16 * s + 8 * hf;
      *reinterpret_cast<f32x4*>(dst) = f32x4{t8[0], t8[1], t8[2], t8[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{t8[4], t8[5], t8[6], t8[7]};
    }
  }

  // 4. dkn = P_k^T db, into dKn or added into dK
  const uint16_t* Pk = a.Pk + (int64_t)h * a.P_hs;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rk = 16 * s + 8 * hf + e;
        pa[e] = __builtin_bit_cast(__bf16, rk < a.rank ? Pk[rk * D + 32 * dt + l32] : (uint16_t)0);
      }
      acc = mfma32(pa, dbh[s], acc);
      acc = mfma32(pa, dbl[s], acc);
    }
    if (k_ok) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float* p = (a.dKn_into_dK ? a.dK : a.dKn) + row * D + och(dt, 4 * rg, hf);
        f32x4 v = a.dKn_into_dK ? *reinterpret_cast<f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += acc[4 * rg + e];
        *reinterpret_cast<f32x4*>(p) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key block -> the query blocks that keep it (ascending), per (batch, head).
// A counting sort in 8 slices of query-block rows, one wave each: per-slice
// counts, offsets (each key block's list start, plus the counts of the
// earlier slices), then each wave lists its rows in order. Lists come out
// ascending, and the result does not depend on timing.
// Also the head's key blocks ordered by their number of query blocks, the
// largest first (the dK/dV launch takes them in that order, so the longest
// lists start first and the short ones fill the end; which order equal
// counts take only moves work between compute units, not any result).
// ---------------------------------------------------------------------------
constexpr int kTmWaves = 8;
__global__ __launch_bounds__(64 * kTmWaves) void transpose_map_kernel(const int32_t* __restrict__ idx, int Nq, int Nk,
                                                                     int k, int32_t* __restrict__ tlist,
                                                                     int32_t* __restrict__ toff,
                                                                     int32_t* __restrict__ korder) {
  __shared__ int cnt[kTmWaves][kMaxKeep + 1];
  __shared__ int wsum[kTmWaves];
  __shared__ int kdeg[kMaxKeep];      // query blocks per key block
  __shared__ int dstart[kMaxKeep + 2];  // per count: the first slot of its key blocks
  const int64_t bh = blockIdx.x;
  const int32_t* row0 = idx + bh * (int64_t)Nq * k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NT = 64 * kTmWaves;
  const int r0 = (int)((int64_t)Nq * wv / kTmWaves), r1 = (int)((int64_t)Nq * (wv + 1) / kTmWaves);
  for (int w = 0; w < kTmWaves; ++w)
    for (int c = tid; c <= Nk; c += NT) cnt[w][c] = 0;
  __syncthreads();
  // 1. counts of the wave's slice
  for (int64_t e = (int64_t)r0 * k + lane; e < (int64_t)r1 * k; e += 64) {
    const int c = row0[e];
    if ((unsigned)c < (unsigned)Nk) atomicAdd(&cnt[wv][c], 1);
  }
  __syncthreads();
  // 2. offsets: thread t takes the key blocks [t S, (t + 1) S); an exclusive
  // scan of the segments' totals over the threads gives each segment's start
  const int S = (Nk + NT - 1) / NT;
  const int c0 = min(Nk, tid * S), c1 = min(Nk, c0 + S);
  int seg = 0;
  for (int c = c0; c < c1; ++c)
    for (int w = 0; w < kTmWaves; ++w) seg += cnt[w][c];
  int incl = seg;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int run = incl - seg;
  for (int w = 0; w < wv; ++w) run += wsum[w];
  for (int c = c0; c < c1; ++c) {
    toff[bh * (Nk + 1) + c] = run;
    const int first = run;
    for (int w = 0; w < kTmWaves; ++w) {
      const int n = cnt[w][c];
      cnt[w][c] = run;
      run += n;
    }
    kdeg[c] = run - first;
  }
  for (int d = tid; d <= Nq + 1; d += NT) dstart[d] = 0;
  if (tid == NT - 1) {
    int total = 0;
    for (int w = 0; w < kTmWaves; ++w) total += wsum[w];
    toff[bh * (Nk + 1) + Nk] = total;
  }
  __syncthreads();
  // key blocks by count, the largest first: a bucket per count, the buckets
  // laid out from the largest count down (Nq fits one pass of 512 lanes
  // for the bucket starts, summed from the top)
  for (int c = tid; c < Nk; c += NT) atomicAdd(&dstart[Nq - min(kdeg[c], Nq)], 1);
  __syncthreads();
  if (wv == 0) {  // exclusive scan over the buckets (count Nq first)
    int base = 0;
    for (int d0 = 0; d0 <= Nq; d0 += 64) {
      const int d = d0 + lane;
      const int v = d <= Nq ? dstart[d] : 0;
      int inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
      }
      if (d <= Nq) dstart[d] = base + inc - v;
      base += __shfl(inc, 63);
    }
  }
  __syncthreads();
  for (int c = tid; c < Nk; c += NT) korder[bh * Nk + atomicAdd(&dstart[Nq - min(kdeg[c], Nq)], 1)] = c;
  __syncthreads();
  // 3. each wave lists its slice's rows in order (a row keeps a key block at
  // most once, so one row's atomics never meet on one counter)
  int32_t* out = tlist + bh * (int64_t)Nq * k;
  for (int qb = r0; qb < r1; ++qb) {
    for (int jj = lane; jj < k; jj += 64) {
      const int c = row0[(int64_t)qb * k + jj];
      if ((unsigned)c < (unsigned)Nk) out[atomicAdd(&cnt[wv][c], 1)] = qb;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------------------
// Softmax branch: dQ per query block.
// ---------------------------------------------------------------------------
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, BQ == 128 ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = BQ / 32;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint16_t smem0[TileSmem<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[TileSmem<D>::kElems];
  __shared__ int sidx[kMaxKeep];
  int64_t bh;
  int qb;
  if (!xcd_group_item(blockIdx.x, a.Nq, (int64_t)a.B * a.H, bh, qb)) return;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int tok0 = qb * BQ + wv * 32;
  const int q_tok = tok0 + l32;
  const bool q_ok = q_tok < a.L;
  const int q_cl = min(q_tok, a.L - 1);
  const int q_chunk = q_cl / a.ar_tokens;
  const int key_hi = min(a.L, (q_chunk + 1) * a.ar_tokens);
  const int key_lo = a.ar_window > 0 ? max(0, (q_chunk - a.ar_window + 1) * a.ar_tokens) : 0;
  const int64_t row = ((int64_t)b * a.L + q_cl) * a.H + h;

  u32x4 qreg[D / 16], dreg[D / 16];
  {
    const uint16_t* qp = a.Q + (int64_t)b * a.sq_b + (int64_t)q_cl * a.sq_l + (int64_t)h * a.sq_h;
    const uint16_t* dp = a.dOs + row * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qreg[s] = q_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
      dreg[s] = q_ok ? *reinterpret_cast<const u32x4*>(dp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
    }
  }
  const float lse = q_ok ? a.lse[bh * a.L + q_cl] : INFINITY;
  const float Di = q_ok ? a.Dd[bh * a.L + q_cl] : 0.f;
  f32x16 dqa[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqa[i] = f32x16{};

  const int32_t* irow = a.idx + (bh * a.Nq + qb) * a.kkeep;
  const uint16_t* Kb = a.K + (int64_t)b * a.sk_b + (int64_t)h * a.sk_h;
  const uint16_t* Vb = a.V + (int64_t)b * a.sv_b + (int64_t)h * a.sv_h;
  DirectTileLoader<D, NW> ld;
  ld.init(Kb, a.sk_l, Vb, a.sv_l, a.L, lane, wv);
  for (int i = tid; i < a.kkeep; i += NT) sidx[i] = irow[i];
  __syncthreads();
  auto block_tok0 = [&](int i) {
    const int c = __builtin_amdgcn_readfirstlane(sidx[i]);
    return (unsigned)c < (unsigned)a.Nk ? c * 64 : a.L;
  };
  const int wave_hi = __builtin_amdgcn_readfirstlane(key_hi);
  const int wave_lo = __builtin_amdgcn_readlane(key_lo, 31);
  auto mask_half = [&](f32x16& sacc, int key0, int kt) {
    const int base = key0 + 32 * kt + 4 * hf;
    const int lim_hi = key_hi - base, lim_lo = key_lo - base;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = 8 * (r >> 2) + (r & 3);
      if (o >= lim_hi || o < lim_lo) sacc[r] = -INFINITY;
    }
  };
  // One kept block as two halves of 32 keys, each: S^T and dP^T (two
  // independent MFMA chains), dS^T, then dQ^T += K^T dS^T. Working a half at
  // a time keeps the register count within two waves per SIMD.
  auto compute = [&](const uint16_t* tile, int key0) {
    const uint16_t* Ks = tile;
    const uint16_t* Vs = tile + 64 * D;
    const bool edge = key0 + 64 > wave_hi || key0 < wave_lo;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 sv = {}, pv = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sv = mfma32(lds_u_row<D>(Ks, 32 * kt + l32, 2 * s + hf), as_bf16x8(qreg[s]), sv);
        pv = mfma32(lds_k_chunk<D>(Vs, 32 * kt + l32, 2 * s + hf), as_bf16x8(dreg[s]), pv);
      }
      if (edge) mask_half(sv, key0, kt);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sv[r], a.scale_log2, -lse));
        ds[r] = p * (pv[r] - Di);
      }
      const bf16x8 dsa = to_bf16x8(ds), dsb = to_bf16x8(ds + 8);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) dqa[dt] = mfma32(lds_u_t_operand<D>(Ks, lane, dt, 32 * kt), dsa, dqa[dt]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        dqa[dt] = mfma32(lds_u_t_operand<D>(Ks, lane, dt, 32 * kt + 16), dsb, dqa[dt]);
    }
  };
  // K rows read both ways (u_swz), V rows by rows only (k_swz)
  auto issue = [&](uint16_t* tile, int key0) {
    ld.issue_swz(tile, key0, lane, wv, false, [](int t) { return u_swz<D>(t); });
    ld.issue_swz(tile + 64 * D, key0, lane, wv, true, [](int t) { return k_swz<D>(t); });
  };
  issue(smem0, block_tok0(0));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int it = 0;
  for (; it + 1 < a.kkeep; it += 2) {
    issue(smem1, block_tok0(it + 1));
    compute(smem0, block_tok0(it));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 2 < a.kkeep) issue(smem0, block_tok0(it + 2));
    compute(smem1, block_tok0(it + 1));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (it < a.kkeep) compute(smem0, block_tok0(it));

  if (q_ok) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = och(dt, 4 * rg, hf);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a.sm_scale * dqa[dt][4 * rg + e];
        if (a.dQn_into_dQ) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(a.dQn + row * D + c0);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += x[e];
        }
        *reinterpret_cast<f32x4*>(a.dQ + row * D + c0) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// Softmax branch: dK and dV per key block.
// ---------------------------------------------------------------------------
// Workgroup = 4 waves on one 64-key block, whose K and V tiles are staged in
// LDS once: wave w works on keys 32 (w & 1) .. +31 and on query sub-tile
// (w >> 1) of every 64-query unit; the two waves of a key half add their
// dK^T, dV^T through LDS at the end. Per unit of the query blocks that keep
// the key block, the Q and dO_s rows (read by rows and transposed, so kept
// with the u_swz chunk swizzle) and the unit's 64 log-sum-exp and D values
// (4 bytes a lane) are staged with direct-to-LDS loads; the tiles stay small
// (64.5 KB) so that two workgroups share a compute unit and one's loads
// overlap the other's matrix work.
template <int D, int BQ>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int UPB = BQ / 64;  // 64-query units per query block
  __shared__ __attribute__((aligned(16))) uint16_t qd[2 * 64 * D];  // Q then dO_s rows of the unit
  __shared__ __attribute__((aligned(16))) uint16_t kv[2 * 64 * D];  // K then V rows of the key block
  __shared__ __attribute__((aligned(16))) float rowv[2][64];        // lse, D of the unit
  int64_t bh;
  int kb;
  // the head's key blocks in the order of korder (the longest query lists
  // first); consecutive workgroups go to consecutive XCDs
  {
    const int64_t n = blockIdx.x;
    bh = n / a.Nk;
    kb = a.korder[n];
  }
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int kh = wv & 1, qp = wv >> 1;
  const int krow0 = 32 * kh;  // the wave's first key row in the key tile
  const int k_tok = kb * 64 + krow0 + l32;
  const bool k_ok = k_tok < a.L;
  const int k_cl = min(k_tok, a.L - 1);
  // queries that see this key: [q_lo, q_hi) (q_hi <= L masks the tail)
  const int k_chunk = k_cl / a.ar_tokens;
  const int q_lo = k_chunk * a.ar_tokens;
  const int q_hi = a.ar_window > 0 ? min(a.L, (k_chunk + a.ar_window) * a.ar_tokens) : a.L;
  const int64_t krow = ((int64_t)b * a.L + k_cl) * a.H + h;

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dka[i] = f32x16{};
    dva[i] = f32x16{};
  }
  // the key block's K and V tiles (rows past L read as zeros)
  {
    DirectTileLoader<D, 4> lkv;
    lkv.init(a.K + (int64_t)b * a.sk_b + (int64_t)h * a.sk_h, a.sk_l, a.V + (int64_t)b * a.sv_b + (int64_t)h * a.sv_h,
             a.sv_l, a.L, lane, wv);
    lkv.issue_swz(kv, kb * 64, lane, wv, false, [](int t) { return k_swz<D>(t); });
    lkv.issue_swz(kv + 64 * D, kb * 64, lane, wv, true, [](int t) { return k_swz<D>(t); });
  }
  DirectTileLoader<D, 4> ld;
  ld.init(a.Q + (int64_t)b * a.sq_b + (int64_t)h * a.sq_h, a.sq_l, a.dOs + (int64_t)b * a.L * a.H * D + (int64_t)h * D,
          (int64_t)a.H * D, a.L, lane, wv);
  // head-major rows of lse and D: 4 bytes per lane, one wave each
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.lse + bh * a.L), 0, a.L * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.Dd + bh * a.L), 0, a.L * 4, 0x00020000);
  const int32_t* list = a.tlist + bh * (int64_t)a.Nq * a.kkeep;
  const int e0 = a.toff[bh * (a.Nk + 1) + kb], e1 = a.toff[bh * (a.Nk + 1) + kb + 1];
  const uint16_t* Ks = kv;
  const uint16_t* Vs = kv + 64 * D;
  const uint16_t* Qs = qd;
  const uint16_t* Ds = qd + 64 * D;
  const int n_units = (e1 - e0) * UPB;
  // the query block of the next unit is read right after this unit's tile
  // loads are issued, so that it arrives with them instead of holding up the
  // next unit's loads (the barriers' waits would take it in before them)
  int qb_next = n_units > 0 ? list[e0] : 0;
  for (int u = 0; u < n_units; ++u) {
    const int q0 = __builtin_amdgcn_readfirstlane(qb_next) * BQ + 64 * (u % UPB);
    __syncthreads();  // the previous unit's readers are done
    ld.issue_swz(qd, q0, lane, wv, false, [](int t) { return u_swz<D>(t); });
    ld.issue_swz(qd + 64 * D, q0, lane, wv, true, [](int t) { return u_swz<D>(t); });
    if (wv < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wv ? drs : lrs, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) float*)rowv[wv]),
          4, 4 * lane, (unsigned)q0 * 4, 0, 0);
    if (u + 1 < n_units) qb_next = list[e0 + (u + 1) / UPB];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int qr0 = 32 * qp;  // first row of the wave's sub-tile in the unit
    f32x16 sa = {}, pa = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 qa = lds_u_row<D>(Qs, qr0 + l32, 2 * s + hf);
      const bf16x8 da = lds_u_row<D>(Ds, qr0 + l32, 2 * s + hf);
      sa = mfma32(qa, lds_k_chunk<D>(Ks, krow0 + l32, 2 * s + hf), sa);
      pa = mfma32(da, lds_k_chunk<D>(Vs, krow0 + l32, 2 * s + hf), pa);
    }
    // register r holds query row qr0 + 8 (r / 4) + 4 hf + r % 4 of key l32
    float pr[16], dsr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = qr0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      const int q = q0 + qi;
      float p = __builtin_amdgcn_exp2f(fmaf(sa[r], a.scale_log2, -rowv[0][qi]));
      p = (q >= q_lo && q < q_hi) ? p : 0.f;
      pr[r] = p;
      dsr[r] = p * (pa[r] - rowv[1][qi]);
    }
    const bf16x8 p0 = to_bf16x8(pr), p1 = to_bf16x8(pr + 8);
    const bf16x8 s0 = to_bf16x8(dsr), s1 = to_bf16x8(dsr + 8);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      dva[dt] = mfma32(lds_u_t_operand<D>(Ds, lane, dt, qr0), p0, dva[dt]);
      dka[dt] = mfma32(lds_u_t_operand<D>(Qs, lane, dt, qr0), s0, dka[dt]);
      dva[dt] = mfma32(lds_u_t_operand<D>(Ds, lane, dt, qr0 + 16), p1, dva[dt]);
      dka[dt] = mfma32(lds_u_t_operand<D>(Qs, lane, dt, qr0 + 16), s1, dka[dt]);
    }
  }
  if (n_units == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the K/V tile loads
  // the two waves of each key half add their sums: waves 2, 3 hand theirs
  // over through the unit's tile memory, dK^T first, then dV^T
  // (lane-minor: the 64 lanes of a wave write 64 consecutive floats)
  float* red = reinterpret_cast<float*>(qd);
  static_assert(2 * 64 * (D / 2) * 4 <= 2 * 64 * D * 2, "reduction buffer exceeds the staged tiles");
  const int ridx = kh * (D / 2) * 64 + lane;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    if (qp == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[ridx + (16 * dt + r) * 64] = pass ? dva[dt][r] : dka[dt][r];
    }
    __syncthreads();
    if (qp == 0 && k_ok) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            const float sum = (pass ? dva[dt][r] : dka[dt][r]) + red[ridx + (16 * dt + r) * 64];
            v[e] = pass ? sum : a.sm_scale * sum;
          }
          *reinterpret_cast<f32x4*>((pass ? a.dV : a.dK) + krow * D + och(dt, 4 * rg, hf)) = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static int64_t group_grid(int items, int64_t groups) {
  return (int64_t)kNumXcd * ((items + kNumXcd - 1) / kNumXcd) * groups;
}

hipError_t launch_bwd_query(const BwdArgs& a, int D, hipStream_t stream) {
  const dim3 grid((unsigned)group_grid((a.L + 127) / 128, (int64_t)a.B * a.H));
  if (D == 128)
    hipLaunchKernelGGL(bwd_query_kernel<128>, grid, dim3(256), 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL(bwd_query_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_key(const BwdArgs& a, int D, hipStream_t stream) {
  const dim3 grid((unsigned)group_grid((a.L + 127) / 128, (int64_t)a.B * a.H));
  if (D == 128)
    hipLaunchKernelGGL(bwd_key_kernel<128>, grid, dim3(256), 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL(bwd_key_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int D, hipStream_t stream) {
  const dim3 grid((unsigned)group_grid(a.Nq, (int64_t)a.B * a.H));
  if (D == 128 && a.block_q == 128)
    hipLaunchKernelGGL((bwd_dq_kernel<128, 128>), grid, dim3(256), 0, stream, a);
  else if (D == 128 && a.block_q == 64)
    hipLaunchKernelGGL((bwd_dq_kernel<128, 64>), grid, dim3(128), 0, stream, a);
  else if (D == 64 && a.block_q == 128)
    hipLaunchKernelGGL((bwd_dq_kernel<64, 128>), grid, dim3(256), 0, stream, a);
  else if (D == 64 && a.block_q == 64)
    hipLaunchKernelGGL((bwd_dq_kernel<64, 64>), grid, dim3(128), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int D, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.Nk * a.B * a.H));
  if (D == 128 && a.block_q == 128)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 128>), grid, dim3(256), 0, stream, a);
  else if (D == 128 && a.block_q == 64)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 64>), grid, dim3(256), 0, stream, a);
  else if (D == 64 && a.block_q == 128)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, 128>), grid, dim3(256), 0, stream, a);
  else if (D == 64 && a.block_q == 64)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, 64>), grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_transpose_map(const int32_t* idx, int BH, int Nq, int Nk, int k, int32_t* tlist, int32_t* toff,
                                int32_t* korder,
                                hipStream_t stream) {
  if (Nk > kMaxKeep) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_map_kernel, dim3(BH), dim3(64 * kTmWaves), 0, stream, idx, Nq, Nk, k, tlist, toff,
                     korder);
  return hipGetLastError();
}

hipError_t launch_token_outer(const float* X, const float* Yf, const uint16_t* Yb, int64_t y_sb, int64_t y_sl,
                              int64_t y_sh, int B, int H, int L, int D, const RunGeo& runs, float* part,
                              hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)runs.n_runs * B * H));
  if (D == 128)
    hipLaunchKernelGGL(token_outer_kernel<128>, grid, dim3(256), 0, stream, X, Yf, Yb, y_sb, y_sl, y_sh, B, H, L,
                       runs, part);
  else if (D == 64)
    hipLaunchKernelGGL(token_outer_kernel<64>, grid, dim3(256), 0, stream, X, Yf, Yb, y_sb, y_sl, y_sh, B, H, L,
                       runs, part);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dstate_finalize(const float* part, int BH, const RunGeo& runs, int n_ar, int window, int D,
                                  float* dC, uint16_t* dCt_hi, uint16_t* dCt_lo, hipStream_t stream) {
  const int64_t total = (int64_t)BH * n_ar * 32 * D;
  hipLaunchKernelGGL(dstate_finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part,
                     (int64_t)BH, runs, n_ar, window, D, dC, dCt_hi, dCt_lo);
  return hipGetLastError();
}

hipError_t launch_dproj_finalize(const float* part, int B, int H, int n_runs, int rank, int D, bool per_head,
                                 float* dP, hipStream_t stream) {
  const int64_t total = (int64_t)(per_head ? H : 1) * rank * D;
  hipLaunchKernelGGL(dproj_finalize_kernel, dim3((unsigned)((total + 63) / 64)), dim3(256), 0, stream, part, B, H,
                     n_runs, rank, D, per_head ? 1 : 0, dP);
  return hipGetLastError();
}

hipError_t launch_dgate(const float* dg_head, int B, int L, int H, int64_t g_sb, int64_t g_sl, int64_t g_sh,
                        float* dg, hipStream_t stream) {
  const int64_t total = (int64_t)(g_sb ? B : 1) * (g_sl ? L : 1) * (g_sh ? H : 1);
  hipLaunchKernelGGL(dgate_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, dg_head, B, L, H,
                     g_sb, g_sl, g_sh, dg);
  return hipGetLastError();
}

}  // namespace sd
