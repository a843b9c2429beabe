// One streaming pass over K, V that prepares the fused layer: the block
// means of K (for the block scores) and the partial low-rank states
// C = sum_j k~_j v_j^T (robotworld.top SparkDiffusion write-up, section 2.1:
// top-k over block-level scores; k~_j = R_r(p_j) phi(P_k kn_j), RoPE after
// phi; C linear in the sequence length).
//
// One workgroup (4 waves) owns a run of 64-token tiles of one (batch, head),
// aligned to query blocks. Per tile:
//   * Kn and V tiles are staged into LDS with raw buffer loads (double
//     buffered, the next tile in flight during the current one);
//   * waves 0-1 project 32 tokens each onto the rank dims with P_k on MFMA,
//     apply phi, and park k~ in an LDS patch, while waves 2-3 sum the staged
//     K tile's columns in float64 (exact for bf16 values) for the key-block
//     means; all threads rotate the RoPE pairs; each wave then owns 32
//     channels of C^T and accumulates V^T k~ on MFMA (V^T operands from
//     transposing LDS reads, k~ split into bf16 hi + lo parts).
// K and V are each read from HBM once. (The query-block means come from the
// pooling kernel, which streams Q once.)
#include "sd_device.h"
#include "sd_launch.h"
#include "sd_tiles.h"

namespace sd {

__device__ __forceinline__ float phi_elu1_p(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <int D>
__global__ __launch_bounds__(256) void prepare_stream_kernel(PrepareArgs a) {
  constexpr int NW = 4;
  constexpr int CH = D / 64;  // channels per lane in the K block sums
  __shared__ __attribute__((aligned(16))) uint16_t tile0[TileSmem<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[TileSmem<D>::kElems];
  __shared__ float F[64 * 33];
  __shared__ double kred[D];

  // All heads of a run of tokens run side by side, so that together the
  // workgroups read whole token rows of K and V (DRAM-friendly).
  const int64_t nbh = (int64_t)a.B * a.H;
  const int64_t bh = blockIdx.x % nbh;
  const int chunk = (int)(blockIdx.x / nbh);
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int ntiles = (a.L + 63) / 64;
  const int t_begin = chunk * a.chunk_tiles;
  const int t_end = min(ntiles, t_begin + a.chunk_tiles);
  const int hw = a.Hg * a.Wg;

  const uint16_t* Knb = a.Kn + (int64_t)b * a.sk_b + (int64_t)h * a.sk_h;
  const uint16_t* Vb = a.V + (int64_t)b * a.sv_b + (int64_t)h * a.sv_h;
  // the K tile is staged for the block sums too; when the low-rank branch
  // reads a separate Kn, the sums come from the pooling kernel instead
  const bool pool_k = a.kmean != nullptr;

  DirectTileLoader<D, NW> ld;
  ld.init(Knb, a.sk_l, Vb, a.sv_l, a.L, lane, wv);

  u32x4 P[D / 16];
  {
    const uint16_t* Pk = a.Pk + (int64_t)h * a.P_hs;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      P[s] = (wv < 2 && l32 < a.rank) ? *reinterpret_cast<const u32x4*>(Pk + l32 * D + 16 * s + 8 * hf)
                                      : u32x4{0, 0, 0, 0};
  }
  f32x16 cacc = {};

  if (t_begin < t_end) ld.issue(tile0, t_begin * 64, lane, wv);
  for (int tl = t_begin; tl < t_end; ++tl) {
    const int tok0 = tl * 64;
    uint16_t* cur = ((tl - t_begin) & 1) ? tile1 : tile0;
    uint16_t* nxt = ((tl - t_begin) & 1) ? tile0 : tile1;

    // RoPE factors of this lane's token for the pairs of this wave (issued
    // early so their latency overlaps the projections)
    constexpr int kMaxPW = kMaxRopePairs / NW;
    float2 cs[kMaxPW];
    const int rtok = tok0 + lane;
    {
      const int tc = min(rtok, a.L - 1);
      const int pos[3] = {tc / hw, (tc / a.Wg) % a.Hg, tc % a.Wg};
#pragma unroll
      for (int j = 0; j < kMaxPW; ++j) {
        const int m = wv + NW * j;
        if (m < a.rope.n) {
          const int axis = a.rope.axis[m];
          cs[j] = a.rope_tab[m * a.rope.max_ext + (axis == 0 ? pos[0] : axis == 1 ? pos[1] : pos[2])];
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile `cur` is in; last tile's readers are done
    if (tl + 1 < t_end) ld.issue(nxt, tok0 + 64, lane, wv);

    double ks[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) ks[c] = 0.0;
    const int c0 = lane * CH;
    if (wv < 2) {
      // low-rank features of 32 tokens per wave
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        acc = mfma32(as_bf16x8(P[s]), lds_k_chunk<D>(cur, 32 * wv + l32, 2 * s + hf), acc);
      const bool tok_ok = tok0 + 32 * wv + l32 < a.L;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ri = 8 * (r >> 2) + 4 * hf + (r & 3);
        F[(32 * wv + l32) * 33 + ri] = (ri < a.rank && tok_ok) ? phi_elu1_p(acc[r]) : 0.f;
      }
    } else if (pool_k) {
      // exact float64 block sums of K: wave 2 rows 0..31, wave 3 rows 32..63,
      // CH channels per lane (rows past L were loaded as zeros)
#pragma unroll 8
      for (int t = 32 * (wv - 2); t < 32 * (wv - 1); ++t) {
        const uint16_t* src = cur + t * D + (((c0 >> 3) ^ k_swz<D>(t)) << 3) + (c0 & 7);
        if constexpr (CH == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
          ks[0] += (double)bf16_lo(w);
          ks[1] += (double)bf16_hi(w);
        } else {
          ks[0] += (double)bf16_bits_to_f32(*src);
        }
      }
      if (wv == 3) {
#pragma unroll
        for (int c = 0; c < CH; ++c) kred[c0 + c] = ks[c];
      }
    }
    __syncthreads();
    if (pool_k && wv == 2) {
      const int kb_tok = min(64, a.L - tok0);
#pragma unroll
      for (int c = 0; c < CH; ++c) a.kmean[(bh * a.Nk + tl) * D + c0 + c] = (ks[c] + kred[c0 + c]) / kb_tok;
    }
    // rank-truncated RoPE on the feature patch: lane = token, pairs split over waves
    if (rtok < a.L) {
#pragma unroll
      for (int j = 0; j < kMaxPW; ++j) {
        const int m = wv + NW * j;
        if (m < a.rope.n) {
          float* f = F + lane * 33 + a.rope.dim[m];
          const float u = f[0], v = f[1];
          f[0] = u * cs[j].x - v * cs[j].y;
          f[1] = u * cs[j].y + v * cs[j].x;
        }
      }
    }
    __syncthreads();
    // C^T[d][r] += sum over the tile's tokens of V[tok][d] k~[tok][r]
    if (wv < D / 32) {
      const uint16_t* Vs = cur + 64 * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // token order of the transposing V read: 16s + 4hf + {0..3}, 16s + 8 + 4hf + {0..3}
        float f8[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) f8[p] = F[(16 * s + 8 * (p >> 2) + 4 * hf + (p & 3)) * 33 + l32];
        bf16x8 fhi, flo;
        split_bf16x8(f8, fhi, flo);
        const bf16x8 vop = lds_v_operand<D>(Vs, lane, wv, 16 * s);
        cacc = mfma32(vop, fhi, cacc);
        cacc = mfma32(vop, flo, cacc);
      }
    }
  }
  // partial C of this chunk: lane holds r = l32, channels 32*wv + 8*(r/4) + 4*hf + r%4
  if (wv < D / 32) {
    float* out = a.partial + ((int64_t)bh * a.n_chunks + chunk) * 32 * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) out[l32 * D + 32 * wv + 8 * (r >> 2) + 4 * hf + (r & 3)] = cacc[r];
  }
}

hipError_t launch_prepare_stream(const PrepareArgs& a, int D, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_chunks * a.B * a.H;
  if (D == 128)
    hipLaunchKernelGGL(prepare_stream_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else if (D == 64)
    hipLaunchKernelGGL(prepare_stream_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sd
