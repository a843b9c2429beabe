// One streaming pass over K, V that prepares the fused layer: the block
// means of K (for the block scores) and the partial low-rank states
// C = sum_j k~_j v_j^T (robotworld.top SparkDiffusion write-up, section 2.1:
// top-k over block-level scores; k~_j = R_r(p_j) phi(P_k kn_j), RoPE after
// phi; C linear in the sequence length).
//
// One workgroup (4 waves) owns a run of 64-token tiles of one (batch, head),
// aligned to query blocks; about three workgroups per CU, all resident at
// once. Under a causal window the runs follow the autoregressive chunks
// instead (a run counts only the tokens of its chunk, one partial state per
// chunk run) and the key-block means come from the pooling kernel. Per tile:
//   * each thread prefetches its share of the next tile's K and V rows into
//     registers (buffer loads) and writes them into the LDS tile when the
//     tile's turn comes;
//   * each wave projects 16 tokens onto the rank dims with P_k on MFMA,
//     applies phi, rotates the RoPE pairs in registers, splits the features
//     into bf16 hi + lo parts once and stores them as MFMA operands; it also
//     sums 16 of the tile's K rows in float64 (exact for bf16 values) for
//     the key-block means;
//   * each wave owns 32 channels of C^T and accumulates V^T k~ on MFMA (V^T
//     operands from transposing LDS reads).
// The rank dims are held in slot order: every RoPE pair occupies two
// adjacent slots starting at an even slot, so both features of a pair land
// in one lane of the projection's output; the partial states are written in
// slot order and the finalising sum maps slots back to ranks.
// K and V are each read from HBM once. (The query-block means come from the
// pooling kernel, which streams Q once.)
#include "sd_device.h"
#include "sd_launch.h"
#include "sd_tiles.h"

namespace sd {

typedef double f64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float phi_elu1_p(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// x / d and x % d for 0 <= x < 2^24, d >= 1, with rcp = 1/d rounded to
// float: the float quotient is off by at most one, and one correction step
// each way makes it exact.
__device__ __forceinline__ int div_small(int x, int d, float rcp, int& rem) {
  int q = (int)((float)x * rcp);
  int r = x - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
  rem = r;
  return q;
}

// Register staging of one 64-token K and V tile: thread tid owns 16-byte
// chunk tid % kCpr of rows tid / kCpr + kRows * i.
template <int D>
struct RegTile {
  static constexpr int kCpr = D / 8;              // 16-byte chunks per row
  static constexpr int kPer = 64 * kCpr / 256;    // chunks per thread per tensor
  static constexpr int kRows = 256 / kCpr;        // rows covered by one pass of the workgroup
  static_assert(kRows % 16 == 0, "swizzles must repeat within kRows");
  u32x4 k[kPer], v[kPer];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, unsigned kstr,
                                       unsigned vstr, int tok0, int tid) {
    const int row = tid / kCpr, col = tid % kCpr;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           kr, (int)(row * kstr + 16 * col), (int)((tok0 + kRows * i) * kstr), 0));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           vr, (int)(row * vstr + 16 * col), (int)((tok0 + kRows * i) * vstr), 0));
  }
  // Both swizzles depend on the row only through bits that kRows leaves
  // unchanged, so the LDS addresses of the chunks differ by constants.
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
    const int row = tid / kCpr, col = tid % kCpr;
    uint16_t* kd = tile + row * D + ((col ^ k_swz<D>(row)) * 8);
    uint16_t* vd = tile + 64 * D + row * D + ((col ^ v_swz<D>(row)) * 8);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      *reinterpret_cast<u32x4*>(kd + kRows * i * D) = k[i];
      *reinterpret_cast<u32x4*>(vd + kRows * i * D) = v[i];
    }
  }
};

// Feature operands of the C^T update, bf16 [32 slots][64 tokens]: row j
// holds in its 16-byte chunk 2s + h the tokens 16s + 4h + {0..3} and
// 16s + 8 + 4h + {0..3} (the key order of the transposing V read), chunk c
// stored at c ^ ((j / 2) % 8) so that 16 rows read one chunk column without
// bank conflicts.
__device__ __forceinline__ int fop_index(int j, int t) {
  const int s = t >> 4, u = t & 15;
  const int c = 2 * s + ((u >> 2) & 1);
  const int e = (u & 3) + 4 * (u >> 3);
  return j * 64 + ((c ^ ((j >> 1) & 7)) << 3) + e;
}

template <int D, bool POOL>
__global__ __launch_bounds__(256, 3) void prepare_stream_kernel(PrepareArgs a) {
  constexpr int CH = D / 64;
  constexpr int kFop = 32 * 64;  // elements of one feature operand array
  __shared__ __attribute__((aligned(16))) uint16_t tile[TileSmem<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t Fop[2 * kFop];  // feature operands: hi, then lo
  __shared__ double kred[4 * D];                                  // block-sum partials of the 4 waves
  __shared__ __attribute__((aligned(16))) uint16_t Ps[32 * D];

  // All heads of a run of tokens run side by side, so that together the
  // workgroups read whole token rows of K and V (DRAM-friendly).
  const int64_t nbh = (int64_t)a.B * a.H;
  const int64_t bh = blockIdx.x % nbh;
  const int run = (int)(blockIdx.x / nbh);
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  int t_begin, t_end, tok_lo, tok_hi;  // tiles of the run, tokens of its chunk
  run_extent(a.runs, a.L, run, t_begin, t_end, tok_lo, tok_hi);
  const int hw = a.Hg * a.Wg;

  const uint16_t* Knb = a.Kn + (int64_t)b * a.sk_b + (int64_t)h * a.sk_h;
  const uint16_t* Vb = a.V + (int64_t)b * a.sv_b + (int64_t)h * a.sv_h;
  // POOL: the K tile is summed for the block means too (when the low-rank
  // branch reads a separate Kn, the means come from the pooling kernel)
  constexpr bool pool_k = POOL;
  const unsigned kstr = (unsigned)(a.sk_l * 2), vstr = (unsigned)(a.sv_l * 2);
  // rows past L read as zeros (range-checked buffers); the empty buffers
  // serve loads past the workgroup's run
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)Knb, 0, (int)((a.L - 1) * kstr + 2 * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, (int)((a.L - 1) * vstr + 2 * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t kr0 = __builtin_amdgcn_make_buffer_rsrc((void*)Knb, 0, 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr0 = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, 0, 0x00020000);

  // P_k rows in slot order (empty slots zero), laid out like a K tile
  {
    const uint16_t* Pk = a.Pk + (int64_t)h * a.P_hs;
    for (int c = tid; c < 32 * (D / 8); c += 256) {
      const int row = c / (D / 8), col = c % (D / 8);
      const int rk = a.slot_rank[row];
      *reinterpret_cast<u32x4*>(Ps + row * D + ((col ^ k_swz<D>(row)) * 8)) =
          rk >= 0 ? *reinterpret_cast<const u32x4*>(Pk + rk * D + 8 * col) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 cacc = {};

  // K block sums: wave wv sums rows 16 wv .. +15, lane = CH adjacent
  // channels (the K swizzle of row 16 wv + t depends on t only)
  const int c0 = lane * CH;

  // Projection layout (16x16x32 MFMA): lane (token 16 wv + l16, group g)
  // holds slots 16 rh + 4 g + {0..3}, i.e. slot pairs 8 rh + 2 g + q. Per
  // lane, the RoPE table row and axis of those 4 slot pairs (j = 2 rh + q);
  // slot pairs without a RoPE pair rotate by the identity.
  const int l16 = lane & 15, g = lane >> 4;
  int cs_row[4], cs_axis[4];
  bool cs_on[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 8 * (j >> 1) + 2 * g + (j & 1);
    int m = -1;
#pragma unroll
    for (int pp = 0; pp < 16; ++pp) m = pp == p ? a.slot_pair[pp] : m;
    cs_on[j] = m >= 0;
    m = max(m, 0);
    int ax = 0;
#pragma unroll
    for (int mm = 0; mm < kMaxRopePairs; ++mm) ax = mm == m ? a.rope.axis[mm] : ax;
    cs_row[j] = m * a.rope.max_ext;
    cs_axis[j] = ax;
  }
  // cos/sin of those pairs at this lane's token of the tile at tok0
  auto load_cs = [&](float2(&cs)[4], int tok0) __attribute__((always_inline)) {
    const int tc = min(tok0 + 16 * wv + l16, a.L - 1);
    int pos[3], rest;
    pos[0] = div_small(tc, hw, a.rcp_hw, rest);
    pos[1] = div_small(rest, a.Wg, a.rcp_wg, pos[2]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      cs[j] = a.rope_tab[cs_row[j] + (cs_axis[j] == 0 ? pos[0] : cs_axis[j] == 1 ? pos[1] : pos[2])];
  };

  // One 64-token tile (its key-block partial sums are left in kred, read
  // after the next step's first barrier).
  auto step = [&](RegTile<D>& rt, int tl, float2(&cs)[4], auto&& after_first_barrier) __attribute__((always_inline)) {
    const int tok0 = tl * 64;
    __syncthreads();  // the previous tile's readers are done with the tile
    after_first_barrier();
    rt.store(tile, tid);
    // refill the registers with tile tl + 1; past the run the loads go to
    // empty buffers (zeros, no memory access), so every path issues the
    // same loads and the waits stay counted
    const bool more = tl + 1 < t_end;
    rt.load(more ? kr : kr0, more ? vr : vr0, kstr, vstr, (tl + 1) * 64, tid);
    __syncthreads();

    {
      // k~ of tokens 16 wv .. +15: phi(P_k k) on 16x16x32 MFMAs (both
      // 16-slot halves), the RoPE pairs rotated in registers (a pair sits in
      // one lane), split into bf16 hi + lo once and stored as the operands of
      // the C^T update; empty slots and tokens past L are zero
      f32x4 acc[2] = {};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const bf16x8 kop = lds_k_chunk<D>(tile, 16 * wv + l16, 4 * s + g);
#pragma unroll
        for (int rh = 0; rh < 2; ++rh)
          acc[rh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_k_chunk<D>(Ps, 16 * rh + l16, 4 * s + g), kop,
                                                            acc[rh], 0, 0, 0);
      }
      const int tk = 16 * wv + l16;
      const bool tok_ok = tok0 + tk >= tok_lo && tok0 + tk < tok_hi;
      uint16_t fh[8], fl[8];
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sl = 16 * rh + 4 * g + e;
          f[e] = (tok_ok && ((a.slot_mask >> sl) & 1u)) ? phi_elu1_p(acc[rh][e]) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int j = 2 * rh + q;
          if (cs_on[j]) {
            const float u = f[2 * q], v = f[2 * q + 1];
            f[2 * q] = u * cs[j].x - v * cs[j].y;
            f[2 * q + 1] = u * cs[j].y + v * cs[j].x;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 hi = (__bf16)f[e];
          const __bf16 lo = (__bf16)(f[e] - (float)hi);
          fh[4 * rh + e] = __builtin_bit_cast(uint16_t, hi);
          fl[4 * rh + e] = __builtin_bit_cast(uint16_t, lo);
        }
      }
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ix = fop_index(16 * rh + 4 * g + e, tk);
          Fop[ix] = fh[4 * rh + e];
          Fop[kFop + ix] = fl[4 * rh + e];
        }
    }
    __syncthreads();
    // C^T[d][slot] += sum over the tile's tokens of V[tok][d] k~[tok][slot],
    // and (POOL) the exact float64 sums of K rows 16 wv .. 16 wv + 15 (rows
    // past L were loaded as zeros): a quarter of the rows after each pair of
    // MFMAs, so that the sums run under them. The tile stays in LDS until the
    // next step's first barrier, and the partials are read after it.
    const bool ct_wave = D / 32 >= 4 || wv < D / 32;  // d = 128: every wave
    const uint16_t* Vs = tile + 64 * D;
    const uint16_t* Fh = Fop;
    const uint16_t* Fl = Fop + kFop;
    const uint16_t* rows = tile + 16 * wv * D;
    double ks[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) ks[c] = 0.0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (ct_wave) {
        const int off = l32 * 64 + (((2 * s + hf) ^ ((l32 >> 1) & 7)) << 3);
        const bf16x8 fhi = as_bf16x8(*reinterpret_cast<const u32x4*>(Fh + off));
        const bf16x8 flo = as_bf16x8(*reinterpret_cast<const u32x4*>(Fl + off));
        const bf16x8 vop = lds_v_operand<D>(Vs, lane, wv, 16 * s);
        cacc = mfma32(vop, fhi, cacc);
        cacc = mfma32(vop, flo, cacc);
      }
      if constexpr (pool_k) {
#pragma unroll
        for (int t = 4 * s; t < 4 * s + 4; ++t) {
          if constexpr (CH == 2) {
            const uint32_t w =
                *reinterpret_cast<const uint32_t*>(rows + t * D + (((c0 >> 3) ^ k_swz<D>(t)) << 3) + (c0 & 7));
            ks[0] += (double)bf16_lo(w);
            ks[1] += (double)bf16_hi(w);
          } else {
            ks[0] += (double)bf16_bits_to_f32(rows[t * D + (((c0 >> 3) ^ k_swz<D>(t)) << 3) + (c0 & 7)]);
          }
        }
      }
    }
    if constexpr (pool_k) {
#pragma unroll
      for (int c = 0; c < CH; ++c) kred[wv * D + c0 + c] = ks[c];
    }
    // the next tile's RoPE factors (kred is rewritten only after the next
    // step's two barriers)
    load_cs(cs, tok0 + 64);
  };

  // The key-block means go out in groups of 4 tiles: wave w finishes the
  // means of the group's tile w (CH channels per lane, a full block divides
  // by 64 exactly as a multiplication) and holds them until the group's
  // last step, then every wave stores its tile's row with one instruction.
  RegTile<D> rt;
  rt.load(kr, vr, kstr, vstr, t_begin * 64, tid);
  float2 cs[4];
  load_cs(cs, t_begin * 64);
  double km[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) km[c] = 0.0;
  const int c0k = lane * CH;
  auto store_means = [&](int tl) __attribute__((always_inline)) {
    double* dst = a.kmean + (bh * a.Nk + tl) * D + c0k;
    if constexpr (CH == 2) {
      *reinterpret_cast<f64x2*>(dst) = f64x2{km[0], km[1]};
    } else {
      dst[0] = km[0];
    }
  };
  // the means of tile tl from the partials in kred (after a barrier that
  // follows their writes)
  auto finish_means = [&](int tl) __attribute__((always_inline)) {
    const int pos = (tl - t_begin) & 3;
    if (pos == wv) {
      const int kb_tok = min(64, a.L - tl * 64);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int cc = c0k + c;
        const double sum = ((kred[cc] + kred[D + cc]) + kred[2 * D + cc]) + kred[3 * D + cc];
        km[c] = kb_tok == 64 ? sum * 0.015625 : sum / kb_tok;
      }
    }
    if (pos == 3) store_means(tl - 3 + wv);
  };
  for (int tl = t_begin; tl < t_end; ++tl) {
    step(rt, tl, cs, [&]() __attribute__((always_inline)) {
      if constexpr (pool_k) {
        if (tl > t_begin) finish_means(tl - 1);
      }
    });
  }
  if constexpr (pool_k) {
    __syncthreads();
    if (t_end > t_begin) finish_means(t_end - 1);
    const int rem = (t_end - t_begin) & 3;  // tiles of the last, unfinished group
    if (rem != 0 && wv < rem) store_means(t_end - rem + wv);
  }
  // partial C of this run in slot order: lane holds slot l32, channels
  // 32 wv + 8 (r / 4) + 4 hf + r % 4
  if (wv < D / 32) {
    float* out = a.partial + ((int64_t)bh * a.runs.n_runs + run) * 32 * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) out[l32 * D + 32 * wv + 8 * (r >> 2) + 4 * hf + (r & 3)] = cacc[r];
  }
}

hipError_t launch_prepare_stream(const PrepareArgs& a, int D, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.runs.n_runs * a.B * a.H));
  const bool pool = a.kmean != nullptr;
  if (D == 128 && pool)
    hipLaunchKernelGGL((prepare_stream_kernel<128, true>), grid, dim3(256), 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL((prepare_stream_kernel<128, false>), grid, dim3(256), 0, stream, a);
  else if (D == 64 && pool)
    hipLaunchKernelGGL((prepare_stream_kernel<64, true>), grid, dim3(256), 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL((prepare_stream_kernel<64, false>), grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sd
