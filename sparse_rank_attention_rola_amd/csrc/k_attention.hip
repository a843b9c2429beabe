// Block-sparse softmax attention (A_M), the per-token low-rank query output
// and the fused RoLA layer.
//
// robotworld.top SparkDiffusion write-up, section 2.1: A~ = A_M + g (.) C_psi.
// A_M is softmax attention restricted to the kept 1-s of the key blocks of
// each query block; the compensation branch gives O_lr,i = RMSNorm(q~_i^T C)
// with q~_i = R_r(p_i) phi(P_q qn_i); the fusion is O_i = O_s,i + g_i r_i
// O_lr,i with r_i the RMS of O_s,i. Section 4 (autoregressive extension):
// both branches may be restricted to a causal window over chunks of tokens;
// a query then sees only the keys of its window, in the kept blocks and in
// the state C of its chunk.
//
// One workgroup owns one query block (block_q = 32 * waves queries) of one
// (batch, head); each wave owns 32 queries. All XCDs work on the same head at
// a time, each on a contiguous eighth of its query blocks, so the last-level
// cache holds one head's K/V and each L2 sees spatially close query blocks.
//
// Per kept key block (64 keys):
//   * the K and V tiles are staged through LDS (double buffered: the next
//     block's global loads are in flight while the current block computes);
//   * S^T = K Q^T on 32x32x16 bf16 MFMA: the transposed product puts one
//     query per lane column, so the online-softmax max/sum of a query is a
//     32-register reduction plus one exchange with lane l^32;
//   * P (bf16) feeds O^T += V^T P^T directly from the accumulator registers
//     (keys permuted consistently in both operands), V^T read from the
//     transposed LDS tile.
// The epilogue (fused / low-rank modes) projects the wave's queries with
// P_q on MFMA, applies phi and the rank-truncated RoPE through a small LDS
// patch, multiplies by the head's state C (bf16 hi+lo split of both
// operands, ~16-bit accurate), RMS-normalises per query, and blends.
#include "sd_device.h"
#include "sd_launch.h"
#include "sd_tiles.h"

namespace sd {

enum AttnMode { kModeSparse = 0, kModeLowrank = 1, kModeFused = 2 };

constexpr int kAttnMinWaves = 2;  // waves per SIMD the register budget must allow (block_q = 128)

__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// max(a, b, c) in one v_max3_f32 (the compiler's fmaxf would first quiet each
// MFMA result; scores are never NaN here).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Low-rank query branch for the 32 queries of one wave, in three parts so
// that the features can be formed while the first K/V tile lands:
//   lowrank_load:     the lane's P_q rows (A operands of the projection) and
//                     the cos/sin of its RoPE pairs;
//   lowrank_features: q~ = R(p) phi(P_q qn) through the wave's LDS patch Fw
//                     (32 x 32 floats, feat_at), split into bf16 hi + lo B operands
//                     (lane l32 = query, ranks 16s + 8hf .. +7);
//   lowrank_output:   y = C^T q~ with the state C of the lane's chunk (0
//                     without a causal window), y / sqrt(mean(y^2) + eps) * w
//                     in the O^T accumulator layout.
template <int D>
struct LowrankLoads {
  u32x4 pa[D / 16];
  float2 cs[kMaxRopePairs / 2];
};

template <int D>
__device__ __forceinline__ void lowrank_load(const AttnArgs& a, int h, int tok0, int lane, LowrankLoads<D>& ld) {
  const int hf = lane >> 5, l32 = lane & 31;
  const int tok = tok0 + l32;
  const int hw = a.Hg * a.Wg;
  const int pos[3] = {min(tok / hw, a.rope.max_ext - 1), (tok / a.Wg) % a.Hg, tok % a.Wg};
#pragma unroll
  for (int j = 0; j < kMaxRopePairs / 2; ++j) {
    const int m = 2 * j + hf;
    ld.cs[j] = float2{1.f, 0.f};
    if (2 * j < a.rope.n && m < a.rope.n) {
      // constant offsets into the arguments: scalar loads (a lane-indexed
      // read of the argument block would be a vector load and a wait)
      const int axis = hf ? a.rope.axis[2 * j + 1] : a.rope.axis[2 * j];
      ld.cs[j] = a.rope_tab[m * a.rope.max_ext + (axis == 0 ? pos[0] : axis == 1 ? pos[1] : pos[2])];
    }
  }
  const uint16_t* Pq = a.Pq + (int64_t)h * a.P_hs;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    ld.pa[s] = (l32 < a.rank) ? *reinterpret_cast<const u32x4*>(Pq + l32 * D + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
}

// A wave's feature patch: 32 rows (queries) of 32 floats (ranks), 4 KB. The
// column is XORed with an even value that differs between the 16 rows of
// each parity, so the lanes' rows fall in distinct banks and each even/odd
// column pair stays adjacent. The patches of up to 4 waves (16 KB) fit the
// second tile buffer at every head dimension.
__device__ __forceinline__ int feat_at(int row, int col) { return row * 32 + (col ^ (2 * ((row >> 1) & 15))); }
static_assert(4 * 32 * 32 * 4 <= TileSmem<64>::kElems * 2, "feature patches exceed the tile buffer");

// The patch belongs to one wave: its LDS accesses complete in issue order, so
// the steps below need no barrier between them.
template <int D>
__device__ __forceinline__ void lowrank_features(const u32x4* qn, const AttnArgs& a, const LowrankLoads<D>& ld,
                                                 float* Fw, int lane, bf16x8 (&qhi)[2], bf16x8 (&qlo)[2]) {
  const int hf = lane >> 5, l32 = lane & 31;
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = mfma32(as_bf16x8(ld.pa[s]), as_bf16x8(qn[s]), acc);
  // acc: column = query l32, row = rank index 8*(r/4) + 4*hf + r%4
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ri = 8 * (r >> 2) + 4 * hf + (r & 3);
    Fw[feat_at(l32, ri)] = ri < a.rank ? phi_elu1(acc[r]) : 0.f;
  }
  // RoPE: lane l32 = token; the two lane halves take the even and odd pairs
#pragma unroll
  for (int j = 0; j < kMaxRopePairs / 2; ++j) {
    const int m = 2 * j + hf;
    if (2 * j < a.rope.n && m < a.rope.n) {
      const float2 cs = ld.cs[j];
      const int d0 = hf ? a.rope.dim[2 * j + 1] : a.rope.dim[2 * j];  // scalar loads, as above
      float* f0 = Fw + feat_at(l32, d0);
      float* f1 = Fw + feat_at(l32, d0 + 1);
      const float u = *f0, v = *f1;
      *f0 = u * cs.x - v * cs.y;
      *f1 = u * cs.y + v * cs.x;
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float t8[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) t8[p] = Fw[feat_at(l32, 16 * s + 8 * hf + p)];
    split_bf16x8(t8, qhi[s], qlo[s]);
  }
}

// The state C^T (bf16 hi and lo parts) of chunk c as the A operands of the
// lane: channel 32 dt + l32, ranks 16 s + 8 hf .. + 7.
template <int D>
struct LowrankState {
  u32x4 hi[D / 32][2], lo[D / 32][2];
};

template <int D>
__device__ __forceinline__ void lowrank_state_load(const AttnArgs& a, int b, int h, int c, int lane,
                                                   LowrankState<D>& st) {
  const int hf = lane >> 5, l32 = lane & 31;
  const int n_ar = (a.L + a.ar_tokens - 1) / a.ar_tokens;
  const int64_t base = (((int64_t)b * a.H + h) * n_ar + c) * D * 32 + (int64_t)l32 * 32 + 8 * hf;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      st.hi[dt][s] = *reinterpret_cast<const u32x4*>(a.Ct_hi + base + (int64_t)32 * dt * 32 + 16 * s);
      st.lo[dt][s] = *reinterpret_cast<const u32x4*>(a.Ct_lo + base + (int64_t)32 * dt * 32 + 16 * s);
    }
}

// first: the state of the wave's first chunk, loaded by the caller
template <int D>
__device__ __forceinline__ void lowrank_output(const bf16x8 (&qhi)[2], const bf16x8 (&qlo)[2], const AttnArgs& a,
                                               int b, int h, int q_chunk, int lane, const LowrankState<D>& first,
                                               f32x16 (&out)[D / 32]) {
  const int hf = lane >> 5;
  const int c_first = __builtin_amdgcn_readfirstlane(q_chunk);
  const int c_last = __builtin_amdgcn_readlane(q_chunk, 31);
  // The wave's queries may fall in several autoregressive chunks (the
  // chunk index grows with the token): the product is formed once per chunk
  // with that chunk's state and each lane keeps the one of its own chunk.
  auto product = [&](const LowrankState<D>& st, bool keep) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      f32x16 y = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        y = mfma32(as_bf16x8(st.hi[dt][s]), qhi[s], y);
        y = mfma32(as_bf16x8(st.lo[dt][s]), qhi[s], y);
        y = mfma32(as_bf16x8(st.hi[dt][s]), qlo[s], y);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) out[dt][r] = keep ? y[r] : out[dt][r];
    }
  };
  product(first, true);
  for (int c = c_first + 1; c <= c_last; ++c) {
    LowrankState<D> st;
    lowrank_state_load<D>(a, b, h, c, lane, st);
    product(st, q_chunk == c);
  }
  float ss = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss += out[dt][r] * out[dt][r];
  ss += __shfl_xor(ss, 32);
  const float inv = rsqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float w = inv;
      if (a.rmsw) w *= bf16_bits_to_f32(a.rmsw[32 * dt + 8 * (r >> 2) + 4 * hf + (r & 3)]);
      out[dt][r] *= w;
    }
}

// Stores one lane's 64 (or 32) values of a [B, L, H, D] row in the O^T
// accumulator layout: groups of 4 consecutive channels.
template <int D>
__device__ __forceinline__ void store_row(void* base, bool f32, int64_t off, const f32x16 (&v)[D / 32], int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * dt + 8 * rg + 4 * hf;
      if (f32) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = v[dt][4 * rg + i];
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off + d0) = o;
      } else {
        u32x2 o;
        o[0] = pack_bf16x2(v[dt][4 * rg], v[dt][4 * rg + 1]);
        o[1] = pack_bf16x2(v[dt][4 * rg + 2], v[dt][4 * rg + 3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + off + d0) = o;
      }
    }
}

template <int D, int BQ, int MODE>
__global__ __launch_bounds__(BQ * 2, BQ == 128 ? kAttnMinWaves : 1) void attention_kernel(AttnArgs a) {
  constexpr int NW = BQ / 32;
  constexpr int NT = NW * 64;
  constexpr bool kLoop = MODE != kModeLowrank;
  __shared__ __attribute__((aligned(16))) uint16_t smem0[TileSmem<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[TileSmem<D>::kElems];
  __shared__ int sidx[kMaxKeep];

  int64_t bh;
  int qb;
  if (!xcd_group_item(blockIdx.x, a.Nq, (int64_t)a.B * a.H, bh, qb)) return;
  const int64_t wi = bh * a.Nq + qb;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hf = lane >> 5, l32 = lane & 31;
  const int tok0 = qb * BQ + wv * 32;
  const int q_tok = tok0 + l32;
  const bool q_ok = q_tok < a.L;
  // keys the lane's query may see: [key_lo, key_hi) of its causal window
  // ([0, L) without one); the bounds grow with the token, so the wave's
  // tightest limits are those of its first and last query
  const int q_chunk = min(q_tok, a.L - 1) / a.ar_tokens;
  const int key_hi = min(a.L, (q_chunk + 1) * a.ar_tokens);
  const int key_lo = a.ar_window > 0 ? max(0, (q_chunk - a.ar_window + 1) * a.ar_tokens) : 0;

  // queries in the B-operand layout
  u32x4 qreg[D / 16];
  {
    const uint16_t* qsrc = (MODE == kModeLowrank) ? a.Qn : a.Q;
    const uint16_t* qp = qsrc + (int64_t)b * a.sq_b + (int64_t)q_tok * a.sq_l + (int64_t)h * a.sq_h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qreg[s] = q_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
  }

  // Low-rank branch (fused and low-rank modes): its operands are loaded
  // before the first K/V tile, and the features are formed while that tile
  // lands; their LDS patch is the second tile buffer, which the loop first
  // fills after the tile-0 barrier. The gate value is loaded here too.
  bf16x8 lqh[2], lql[2];
  float gv = 0.f;
  LowrankLoads<D> lld;
  u32x4 qn_reg[D / 16];
  const bool sep_qn = MODE == kModeFused && a.Qn != a.Q;
  if constexpr (MODE != kModeSparse) {
    lowrank_load<D>(a, h, tok0, lane, lld);
    if (sep_qn) {
      const uint16_t* qp = a.Qn + (int64_t)b * a.sq_b + (int64_t)q_tok * a.sq_l + (int64_t)h * a.sq_h;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        qn_reg[s] = q_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
    }
    if constexpr (MODE == kModeFused)
      gv = q_ok ? a.g[(int64_t)b * a.g_sb + (int64_t)q_tok * a.g_sl + (int64_t)h * a.g_sh] : 0.f;
  }
  auto form_features = [&]() __attribute__((always_inline)) {
    if constexpr (MODE != kModeSparse) {
      float* Fw = reinterpret_cast<float*>(smem1) + wv * (32 * 32);
      lowrank_features<D>(sep_qn ? qn_reg : qreg, a, lld, Fw, lane, lqh, lql);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float ltot = 1.f, m_fin = 0.f;
  if constexpr (!kLoop) form_features();

  if constexpr (kLoop) {
    const int32_t* irow = a.idx + wi * a.kkeep;
    const uint16_t* Kb = a.K + (int64_t)b * a.sk_b + (int64_t)h * a.sk_h;
    const uint16_t* Vb = a.V + (int64_t)b * a.sv_b + (int64_t)h * a.sv_h;
    DirectTileLoader<D, NW> ld;
    ld.init(Kb, a.sk_l, Vb, a.sv_l, a.L, lane, wv);
    float m = -INFINITY, lsum = 0.f;

    // first token of a kept block; an index outside [0, Nk) selects nothing
    auto tok_of = [&](int c) __attribute__((always_inline)) { return (unsigned)c < (unsigned)a.Nk ? c * 64 : a.L; };
    // The block row goes to LDS once: reading it there (lgkm counter) never
    // waits on the tile prefetches in flight (vm counter, completed in order).
    for (int i = tid; i < a.kkeep; i += NT) sidx[i] = irow[i];
    __syncthreads();
    auto block_tok0 = [&](int i) __attribute__((always_inline)) { return tok_of(__builtin_amdgcn_readfirstlane(sidx[i])); };

    // One kept block of 64 keys, as two half-tiles of 32 keys. The lane
    // holds 16 of the 32 keys of its query per half-tile.
    auto mask_half = [&](f32x16& sacc, int key0, int kt) {
      // key of register r: key0 + 32 kt + 4 hf + 8 (r / 4) + r % 4, its
      // offset compared as a constant against two per-lane limits
      const int base = key0 + 32 * kt + 4 * hf;
      const int lim_hi = key_hi - base, lim_lo = key_lo - base;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 8 * (r >> 2) + (r & 3);
        if (o >= lim_hi || o < lim_lo) sacc[r] = -INFINITY;
      }
    };
    const int wave_hi = __builtin_amdgcn_readfirstlane(key_hi);
    const int wave_lo = __builtin_amdgcn_readlane(key_lo, 31);
    auto rescale = [&](bool up, float m_new, float rs) {
      if (__ballot(up)) {
        const float alpha = up ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      m = m_new;
      lsum += rs;
    };
    // S^T (32 keys x 32 queries) = K Q^T for both halves, then per half the
    // softmax and O^T += V^T P^T (keys of each 16-key step in the order
    // 4hf+{0..3}, 8+4hf+{0..3} on both operands). Independent accumulators
    // alternate in every MFMA sequence (the two halves' S^T chains; the
    // channel tiles of O^T): no MFMA waits on the result of the one issued
    // just before it.
    // Softmax of one 64-key block in the log2 domain, in two parts: the
    // block's maximum and whether it moves the reference maximum (only when
    // a score exceeds it by more than 8, i.e. P > 256); then, without
    // touching O, the probabilities of each 32-key half as the two bf16 B
    // operands of its PV products (keys 4hf + {0..3}, 8 + 4hf + {0..3} of
    // each 16-key step) and their sum.
    auto block_max = [&](const f32x16& s0, const f32x16& s1, float& m_new) __attribute__((always_inline)) {
      // a v_max3 tree over the 32 scores (depth 4)
      float t[12];
#pragma unroll
      for (int i = 0; i < 5; ++i) t[i] = max3f(s0[3 * i], s0[3 * i + 1], s0[3 * i + 2]);
#pragma unroll
      for (int i = 0; i < 5; ++i) t[5 + i] = max3f(s1[3 * i], s1[3 * i + 1], s1[3 * i + 2]);
      t[10] = s0[15];
      t[11] = s1[15];
      const float u0 = max3f(t[0], t[1], t[2]), u1 = max3f(t[3], t[4], t[5]);
      const float u2 = max3f(t[6], t[7], t[8]), u3 = max3f(t[9], t[10], t[11]);
      float mloc = max3f(u0, u1, max3f(u2, u3, u3));
      mloc = fmaxf(mloc, partner32(mloc, hf)) * a.scale_log2;
      const bool up = mloc > m + 8.f;
      m_new = up ? mloc : m;
      return up;
    };
    auto half_exp = [&](const f32x16& sh, float neg_m, bf16x8& pa, bf16x8& pb) __attribute__((always_inline)) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(sh[r], a.scale_log2, neg_m));
      pa = to_bf16x8(e);
      pb = to_bf16x8(e + 8);
      return sum_bf16x8(pb, sum_bf16x8(pa, 0.f));
    };
    auto compute_kv = [&](const uint16_t* Ks, const uint16_t* Vs, int key0) __attribute__((always_inline)) {
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        s0 = mfma32(lds_k_chunk<D>(Ks, l32, 2 * s + hf), as_bf16x8(qreg[s]), s0);
        s1 = mfma32(lds_k_chunk<D>(Ks, 32 + l32, 2 * s + hf), as_bf16x8(qreg[s]), s1);
      }
      if (key0 + 64 > wave_hi || key0 < wave_lo) {
        mask_half(s0, key0, 0);
        mask_half(s1, key0, 1);
      }
      // The reference maximum m moves only when needed: the probabilities
      // are formed against the current m, and only if a lane has no m yet
      // or a block's row sum shows a score far above m (P up to 2^60 is
      // harmless in bf16 and in the f32 sums) is the block's maximum taken,
      // m moved and the probabilities formed again.
      bf16x8 pa0, pb0, pa1, pb1;
      float rs = 0.f;
      bool redo = __ballot(m == -INFINITY) != 0;
      if (!redo) {
        rs = half_exp(s0, -m, pa0, pb0) + half_exp(s1, -m, pa1, pb1);
        redo = __ballot(!(rs <= 0x1p60f)) != 0;
      }
      if (redo) {
        float m_new;
        const bool up = block_max(s0, s1, m_new);
        rescale(up, m_new, 0.f);
        const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
        rs = half_exp(s0, neg_m, pa0, pb0) + half_exp(s1, neg_m, pa1, pb1);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = mfma32(lds_v_operand<D>(Vs, lane, dt, 0), pa0, oacc[dt]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = mfma32(lds_v_operand<D>(Vs, lane, dt, 16), pb0, oacc[dt]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = mfma32(lds_v_operand<D>(Vs, lane, dt, 32), pa1, oacc[dt]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = mfma32(lds_v_operand<D>(Vs, lane, dt, 48), pb1, oacc[dt]);
      lsum += rs;
    };
    auto compute = [&](const uint16_t* tile, int key0) __attribute__((always_inline)) {
      compute_kv(tile, tile + 64 * D, key0);
    };

    // Double-buffered tiles: block i+1's loads are in flight while block i
    // computes; one wait + barrier per block. The low-rank features are
    // formed while the first block lands.
    ld.issue(smem0, block_tok0(0), lane, wv);
    form_features();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int it = 0;
    for (; it + 1 < a.kkeep; it += 2) {
      ld.issue(smem1, block_tok0(it + 1), lane, wv);
      compute(smem0, block_tok0(it));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (it + 2 < a.kkeep) ld.issue(smem0, block_tok0(it + 2), lane, wv);
      compute(smem1, block_tok0(it + 1));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (it < a.kkeep) {
      compute(smem0, block_tok0(it));
      __syncthreads();
    }
    ltot = lsum + __shfl_xor(lsum, 32);
    m_fin = m;
  }

  const int64_t obase = (int64_t)b * a.so_b + (int64_t)q_tok * a.so_l + (int64_t)h * a.so_h;
  if constexpr (MODE == kModeSparse) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float ss = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        oacc[dt][r] *= inv;
        ss += oacc[dt][r] * oacc[dt][r];
      }
    ss += __shfl_xor(ss, 32);
    if (q_ok) {
      store_row<D>(a.out, a.out_f32, obase, oacc, hf);
      if (a.rms && hf == 0) a.rms[((int64_t)b * a.L + q_tok) * a.H + h] = sqrtf(ss * (1.0f / D));
      // log2-domain log-sum-exp of the query's scaled scores, for the
      // backward's recomputation of P (+inf where the query saw no key)
      if (a.lse && hf == 0) a.lse[((int64_t)b * a.H + h) * a.L + q_tok] = ltot > 0.f ? m_fin + log2f(ltot) : INFINITY;
    }
  } else {
    LowrankState<D> st0;
    lowrank_state_load<D>(a, b, h, __builtin_amdgcn_readfirstlane(q_chunk), lane, st0);
    f32x16 olr[D / 32];
    lowrank_output<D>(lqh, lql, a, b, h, q_chunk, lane, st0, olr);
    if constexpr (MODE == kModeLowrank) {
      if (q_ok) store_row<D>(a.out, a.out_f32, obase, olr, hf);
    } else {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      float ss = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          oacc[dt][r] *= inv;
          ss += oacc[dt][r] * oacc[dt][r];
        }
      ss += __shfl_xor(ss, 32);
      const float rr = sqrtf(ss * (1.0f / D));
      if (a.os_save && q_ok) {
        // the sparse branch's output, RMS and log-sum-exp kept for the backward
        store_row<D>(a.os_save, false, (((int64_t)b * a.L + q_tok) * a.H + h) * D, oacc, hf);
        if (hf == 0) {
          a.rms[((int64_t)b * a.L + q_tok) * a.H + h] = rr;
          a.lse[((int64_t)b * a.H + h) * a.L + q_tok] = ltot > 0.f ? m_fin + log2f(ltot) : INFINITY;
        }
      }
      const float coef = gv * rr;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = fmaf(coef, olr[dt][r], oacc[dt][r]);
      if (q_ok) store_row<D>(a.out, false, obase, oacc, hf);
    }
  }
}

// Explicit instantiation of every variant: the host pass must emit each
// kernel's launch stub.
#define SD_ATTN_INST(D, BQ, MODE) template __global__ void attention_kernel<D, BQ, MODE>(AttnArgs);
#define SD_ATTN_INST_MODES(D, BQ) SD_ATTN_INST(D, BQ, 0) SD_ATTN_INST(D, BQ, 1) SD_ATTN_INST(D, BQ, 2)
SD_ATTN_INST_MODES(128, 128)
SD_ATTN_INST_MODES(128, 64)
SD_ATTN_INST_MODES(64, 128)
SD_ATTN_INST_MODES(64, 64)
#undef SD_ATTN_INST_MODES
#undef SD_ATTN_INST

template <int D, int BQ, int MODE>
static hipError_t launch_attention_t(const AttnArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)kNumXcd * ((a.Nq + kNumXcd - 1) / kNumXcd) * a.B * a.H;
  hipLaunchKernelGGL((attention_kernel<D, BQ, MODE>), dim3((unsigned)grid), dim3(BQ * 2), 0, stream, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_attention_mode(const AttnArgs& a, int D, int BQ, hipStream_t stream) {
  if (D == 128 && BQ == 128) return launch_attention_t<128, 128, MODE>(a, stream);
  if (D == 128 && BQ == 64) return launch_attention_t<128, 64, MODE>(a, stream);
  if (D == 64 && BQ == 128) return launch_attention_t<64, 128, MODE>(a, stream);
  if (D == 64 && BQ == 64) return launch_attention_t<64, 64, MODE>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_attn(const AttnArgs& a, int D, int BQ, hipStream_t stream) {
  return launch_attention_mode<kModeSparse>(a, D, BQ, stream);
}
hipError_t launch_lowrank_query(const AttnArgs& a, int D, int BQ, hipStream_t stream) {
  return launch_attention_mode<kModeLowrank>(a, D, BQ, stream);
}
hipError_t launch_rola_fused(const AttnArgs& a, int D, int BQ, hipStream_t stream) {
  return launch_attention_mode<kModeFused>(a, D, BQ, stream);
}

}  // namespace sd
