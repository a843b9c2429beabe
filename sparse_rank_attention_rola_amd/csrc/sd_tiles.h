// LDS tile staging and the register layouts shared by the attention and
// low-rank kernels (gfx950, wave64, v_mfma_f32_32x32x16_bf16).
//
// MFMA 32x32x16 bf16 operand layout (checked on the hardware):
//   A[i][k]: lane i + 32*(k/8), element k%8      (i < 32, k < 16)
//   B[k][j]: lane j + 32*(k/8), element k%8
//   D[i][j]: lane j + 32*((i/4)%2), register (i/8)*4 + i%4
// With l32 = lane % 32 and hf = lane / 32, the accumulator register r of a
// lane holds row i = 8*(r/4) + 4*hf + r%4 of column j = l32.
//
// A 64-token tile of K (or any [tokens, d] operand read along d) is kept in
// LDS row-major, 16-byte chunk c of row t stored at chunk c ^ (t % 8): the
// 32 lanes that read one chunk column of 32 rows hit distinct banks.
// A 64-token tile of V is kept transposed, Vt[d][token], in 8-byte chunks of
// 4 tokens; chunk c of row d is stored at c ^ f(d), f(d) = (d%16) ^ (d/16),
// which keeps both the transposing stores and the MFMA operand reads free
// of bank conflicts.
#pragma once

#include "sd_device.h"

namespace sd {

template <int D>
struct TileSmem {
  static constexpr int kKElems = 64 * D;  // K tile, bf16
  static constexpr int kVElems = D * 64;  // Vt tile, bf16
  static constexpr int kElems = kKElems + kVElems;
};

__device__ __forceinline__ int vt_swz(int d) { return (d & 15) ^ ((d >> 4) & 15); }

// Global -> registers -> LDS staging of one 64-token tile of K (row-major,
// swizzled) and V (transposed, swizzled) by NT threads.
template <int D, int NT>
struct TileLoader {
  static constexpr int DC = D / 8;              // 16-byte chunks per row
  static constexpr int KPT = 64 * DC / NT;      // K chunks per thread
  static constexpr int VGROUPS = 2 * D;         // (4 tokens x 8 channels) groups per tile
  static constexpr int VPT = (VGROUPS + NT - 1) / NT;
  static_assert(KPT >= 1, "tile too small for the block");

  u32x4 kreg[KPT];
  u32x4 vreg[VPT][4];

  __device__ __forceinline__ void load(const uint16_t* Kb, int64_t sk_l, const uint16_t* Vb, int64_t sv_l,
                                       int tok0, int L, int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int chunk = i * NT + tid;
      const int t = chunk / DC, dc = chunk % DC;
      const int tok = tok0 + t;
      kreg[i] = tok < L ? *reinterpret_cast<const u32x4*>(Kb + (int64_t)tok * sk_l + dc * 8) : u32x4{0, 0, 0, 0};
    }
    if (Vb == nullptr) return;
#pragma unroll
    for (int g = 0; g < VPT; ++g) {
      const int grp = g * NT + tid;
      if (grp < VGROUPS) {
        const int dg = grp % DC, kg = grp / DC;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = tok0 + 4 * kg + j;
          vreg[g][j] = tok < L ? *reinterpret_cast<const u32x4*>(Vb + (int64_t)tok * sv_l + dg * 8)
                               : u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* smem, int tid, bool with_v) const {
    uint16_t* Ks = smem;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int chunk = i * NT + tid;
      const int t = chunk / DC, dc = chunk % DC;
      *reinterpret_cast<u32x4*>(Ks + t * D + ((dc ^ (t & 7)) * 8)) = kreg[i];
    }
    if (!with_v) return;
    uint16_t* Vt = smem + TileSmem<D>::kKElems;
#pragma unroll
    for (int g = 0; g < VPT; ++g) {
      const int grp = g * NT + tid;
      if (grp < VGROUPS) {
        const int dg = grp % DC, kg = grp / DC;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = 8 * dg + i;
          const int w = i >> 1;
          uint32_t e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) e[j] = (i & 1) ? (vreg[g][j][w] >> 16) : (vreg[g][j][w] & 0xFFFFu);
          u32x2 pk;
          pk[0] = e[0] | (e[1] << 16);
          pk[1] = e[2] | (e[3] << 16);
          *reinterpret_cast<u32x2*>(Vt + d * 64 + ((kg ^ vt_swz(d)) * 4)) = pk;
        }
      }
    }
  }
};

// 8 bf16 of K-layout row t (tokens), channels 8*c .. 8*c+7.
template <int D>
__device__ __forceinline__ bf16x8 lds_k_chunk(const uint16_t* Ks, int t, int c) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + t * D + ((c ^ (t & 7)) * 8)));
}

// 4 bf16 of Vt row d, tokens 4*c .. 4*c+3.
__device__ __forceinline__ u32x2 lds_vt_chunk(const uint16_t* Vt, int d, int c) {
  return *reinterpret_cast<const u32x2*>(Vt + d * 64 + ((c ^ vt_swz(d)) * 4));
}

__device__ __forceinline__ bf16x8 cat_bf16x8(u32x2 a, u32x2 b) {
  u32x4 v;
  v[0] = a[0];
  v[1] = a[1];
  v[2] = b[0];
  v[3] = b[1];
  return as_bf16x8(v);
}


// ---------------------------------------------------------------------------
// Direct (global -> LDS) staging of one 64-token K tile and one 64-token V
// tile, both row-major [token][D] bf16. A wave instruction writes 1 KB of
// LDS: lane l's 16 bytes land at base + 16*l, so the swizzle is realised by
// choosing which global 16-byte chunk each lane fetches:
//   K tile: 16-byte chunk c of row t stored at c ^ (t % 8)  (conflict-free
//           reads of one chunk column by 32 consecutive rows);
//   V tile: 16-byte chunk c of row t stored at c ^ 2*(t % 4) (conflict-free
//           transposing reads of 4 rows x 32 bytes per 16-lane group).
// Rows past the end of the sequence are fetched from the last valid row;
// their scores are masked, so they contribute nothing.
template <int D, int NW>
struct DirectTileLoader {
  static constexpr int kSegs = D / 8;          // 1 KB segments per tile
  static constexpr int kSpw = kSegs / NW;      // segments per wave per tile
  static constexpr int kRowBytes = 2 * D;
  static_assert(kSpw >= 1, "tile smaller than the workgroup");

  int koff[kSpw];  // element offset of this lane's K chunk, relative to the tile's first row
  int voff[kSpw];

  __device__ __forceinline__ static void seg_row_chunk(int sg, int lane, int& row, int& p16) {
    const int byte = sg * 1024 + 16 * lane;
    row = byte / kRowBytes;
    p16 = (byte % kRowBytes) / 16;
  }

  __device__ __forceinline__ void init(int lane, int wv, int64_t sk_l, int64_t sv_l) {
#pragma unroll
    for (int i = 0; i < kSpw; ++i) {
      int row, p16;
      seg_row_chunk(wv + NW * i, lane, row, p16);
      koff[i] = row * (int)sk_l + ((p16 ^ (row & 7)) * 8);
      voff[i] = row * (int)sv_l + ((p16 ^ ((row & 3) << 1)) * 8);
    }
  }

  __device__ __forceinline__ void issue(uint16_t* tile, const uint16_t* Kb, int64_t sk_l, const uint16_t* Vb,
                                        int64_t sv_l, int tok0, int L, int lane, int wv) const {
    uint16_t* Ks = tile;
    uint16_t* Vs = tile + 64 * D;
    if (tok0 + 64 <= L) {
      const uint16_t* kb = Kb + (int64_t)tok0 * sk_l;
      const uint16_t* vb = Vb + (int64_t)tok0 * sv_l;
#pragma unroll
      for (int i = 0; i < kSpw; ++i) {
        const int sg = wv + NW * i;
        __builtin_amdgcn_global_load_lds(kb + koff[i], (__attribute__((address_space(3))) void*)(Ks + sg * 512),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + voff[i], (__attribute__((address_space(3))) void*)(Vs + sg * 512),
                                         16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSpw; ++i) {
        const int sg = wv + NW * i;
        int row, p16;
        seg_row_chunk(sg, lane, row, p16);
        const int64_t t = min(tok0 + row, L - 1);
        __builtin_amdgcn_global_load_lds(Kb + t * sk_l + ((p16 ^ (row & 7)) * 8),
                                         (__attribute__((address_space(3))) void*)(Ks + sg * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(Vb + t * sv_l + ((p16 ^ ((row & 3) << 1)) * 8),
                                         (__attribute__((address_space(3))) void*)(Vs + sg * 512), 16, 0, 0);
      }
    }
  }
};

typedef short short4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group,
// lane 4q+k receives element k of the 8-byte chunks addressed by lanes
// q, 4+q, 8+q and 12+q (checked on the hardware).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) uint16_t*)p));
  return __builtin_bit_cast(u32x2, v);
}

// A operand (32 channels x 16 keys) of O^T += V^T P^T from the row-major
// V tile: lane l receives V[kbase + r][32*dt + l%32] for r = 0..3 (first
// read) and V[kbase + 8 + r][...] (second read), kbase = 16*step + 4*(l/32).
template <int D>
__device__ __forceinline__ bf16x8 lds_v_operand(const uint16_t* Vs, int lane, int dt, int key_base) {
  const int G = lane >> 4, j = lane & 15;
  const int r = j >> 2, q = j & 3;
  const int row = key_base + 4 * (G >> 1) + r;       // (row & 3) == r
  const int c8 = 8 * dt + 4 * (G & 1) + q;           // 8-byte chunk of the channel
  const int off = ((c8 >> 1) ^ (r << 1)) * 8 + (c8 & 1) * 4;
  const u32x2 lo = lds_read_tr16(Vs + row * D + off);
  const u32x2 hi = lds_read_tr16(Vs + (row + 8) * D + off);
  return cat_bf16x8(lo, hi);
}

// Largest number of kept key blocks per query block (L <= 131072, 64-key blocks).
constexpr int kMaxKeep = 2048;

// Compile-time description of the rank-truncated 3D RoPE pairs.
constexpr int kMaxRopePairs = 16;
struct RopeArgs {
  int n;
  int max_ext;  // positions per axis in the cos/sin table (max of T, Hg, Wg)
  int dim[kMaxRopePairs];
  int axis[kMaxRopePairs];
};

}  // namespace sd
