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
// LDS has 64 banks of 4 bytes on gfx950. A 64-token tile of K (or any
// [tokens, d] operand read along d) is kept row-major with 16-byte chunk c
// of row t stored at c ^ k_swz(t): the lanes that read one chunk column of
// consecutive rows hit distinct banks. The register-staged loader below keeps
// V transposed, Vt[d][token], in 8-byte chunks of 4 tokens (chunk c of row d
// stored at c ^ f(d), f(d) = (d%16) ^ (d/16)).
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

// 16-byte-chunk swizzle of row t of a row-major K tile: 16 consecutive rows
// (one 16-lane LDS cycle of a b128 read) land on 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int t) {
  return D == 128 ? (t & 15) : ((t >> 1) & 7);  // D = 64: two 128-byte rows share a bank row
}

// 16-byte-chunk swizzle of row t of a row-major V tile read by transposing
// reads: the 4 rows x 64 bytes of one 32-lane LDS cycle hit distinct banks.
template <int D>
__device__ __forceinline__ int v_swz(int t) {
  return D == 128 ? 4 * (t & 3) : 4 * ((t & 3) >> 1);
}

// 16-byte-chunk swizzle of a row-major tile read both ways: by rows (16
// consecutive rows, one chunk column, per 16-lane cycle) and by transposing
// reads (4 consecutive rows x 64 bytes per 32-lane cycle). For d = 128 the
// value is the 4 x 4 transpose of t % 16: bijective on 16 rows, and four
// consecutive rows differ in the chunk group (bits 2, 3). For d = 64 (8
// chunks, two rows per bank row) the 8 rows of one parity among 16 take
// distinct values, and rows t, t + 2 differ in bit 2.
template <int D>
__device__ __forceinline__ int u_swz(int t) {
  return D == 128 ? 4 * (t & 3) + ((t >> 2) & 3) : 4 * ((t >> 1) & 1) + ((t >> 2) & 3);
}

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
      *reinterpret_cast<u32x4*>(Ks + t * D + ((dc ^ k_swz<D>(t)) * 8)) = kreg[i];
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
  return as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + t * D + ((c ^ k_swz<D>(t)) * 8)));
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
// tile, both row-major [token][D] bf16, with raw buffer loads into LDS. A wave
// instruction writes 1 KB of LDS: lane l's 16 bytes land at base + 16*l, so
// the swizzle is realised by choosing which 16-byte chunk each lane fetches:
//   K tile: 16-byte chunk c of row t stored at c ^ k_swz(t);
//   V tile: 16-byte chunk c of row t stored at c ^ v_swz(t).
// The buffer descriptor of each (batch, head) ends at the last valid token,
// so rows past the end of the sequence read as zeros (hardware range check);
// their scores are masked and their zero values contribute nothing.
// Per-load offsets are uniform (SGPR); each lane keeps one 32-bit offset per
// tensor (both swizzles repeat every 16 rows, the distance between a wave's
// consecutive segments when 4 waves share a 128-channel tile).
template <int D, int NW>
struct DirectTileLoader {
  static constexpr int kSegs = D / 8;          // 1 KB segments per tile
  static constexpr int kSpw = kSegs / NW;      // segments per wave per tile
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kRowsPerStep = NW * 1024 / kRowBytes;  // rows between a wave's segments
  static_assert(kSpw >= 1, "tile smaller than the workgroup");

  __amdgpu_buffer_rsrc_t krsrc, vrsrc;
  unsigned kvoff, vvoff;  // byte offsets of this lane's chunks in its first segment
  unsigned kstride, vstride;  // token strides in bytes

  __device__ __forceinline__ static void seg_row_chunk(int sg, int lane, int& row, int& p16) {
    const int byte = sg * 1024 + 16 * lane;
    row = byte / kRowBytes;
    p16 = (byte % kRowBytes) / 16;
  }

  // Kb, Vb: first element of this (batch, head); L valid tokens.
  __device__ __forceinline__ void init(const uint16_t* Kb, int64_t sk_l, const uint16_t* Vb, int64_t sv_l, int L,
                                       int lane, int wv) {
    kstride = (unsigned)(sk_l * 2);
    vstride = (unsigned)(sv_l * 2);
    krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kb, 0, (int)((L - 1) * kstride + 2 * D), 0x00020000);
    vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, (int)((L - 1) * vstride + 2 * D), 0x00020000);
    int row, p16;
    seg_row_chunk(wv, lane, row, p16);
    kvoff = row * kstride + ((p16 ^ k_swz<D>(row)) * 16);
    vvoff = row * vstride + ((p16 ^ v_swz<D>(row)) * 16);
  }

  // K tile of the block starting at token tok0 into Ks (64 x D, swizzled);
  // a tok0 >= L loads nothing but zeros.
  __device__ __forceinline__ void issue_k(uint16_t* Ks, int tok0, int lane, int wv) const {
#pragma unroll
    for (int i = 0; i < kSpw; ++i) {
      const int sg = wv + NW * i;
      unsigned kv = kvoff;
      if constexpr (kRowsPerStep % 16 != 0) {  // the K swizzle does not repeat: recompute
        int row, p16;
        seg_row_chunk(sg, lane, row, p16);
        kv = (row - i * kRowsPerStep) * kstride + ((p16 ^ k_swz<D>(row)) * 16);
      }
      const unsigned rows = (unsigned)(tok0 + i * kRowsPerStep);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krsrc, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint16_t*)(Ks + sg * 512)),
          16, kv, rows * kstride, 0, 0);
    }
  }
  // V tile of the block starting at token tok0 into Vs (64 x D, swizzled).
  __device__ __forceinline__ void issue_v(uint16_t* Vs, int tok0, int wv) const {
#pragma unroll
    for (int i = 0; i < kSpw; ++i) {
      const int sg = wv + NW * i;
      const unsigned rows = (unsigned)(tok0 + i * kRowsPerStep);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrsrc, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint16_t*)(Vs + sg * 512)),
          16, vvoff, rows * vstride, 0, 0);
    }
  }
  // K and V tiles of one block into a tile buffer (K rows, then V rows).
  __device__ __forceinline__ void issue(uint16_t* tile, int tok0, int lane, int wv) const {
    issue_k(tile, tok0, lane, wv);
    issue_v(tile + 64 * D, tok0, wv);
  }
  // The K (second = false) or V (second = true) tile of the block at tok0
  // with the chunk swizzle `swz` of the row (a function of the row that
  // repeats every 16 rows).
  template <class Swz>
  __device__ __forceinline__ void issue_swz(uint16_t* Ts, int tok0, int lane, int wv, bool second, Swz swz) const {
    const __amdgpu_buffer_rsrc_t rs = second ? vrsrc : krsrc;
    const unsigned stride = second ? vstride : kstride;
    int row0, p0;  // the lane's row and slot in the wave's first segment
    seg_row_chunk(wv, lane, row0, p0);
    const unsigned voff0 = (unsigned)row0 * stride + (unsigned)((p0 ^ swz(row0)) * 16);
#pragma unroll
    for (int i = 0; i < kSpw; ++i) {
      const int sg = wv + NW * i;
      unsigned voff = voff0;  // swizzles repeat every 16 rows
      if constexpr (kRowsPerStep % 16 != 0) {
        int row, p16;
        seg_row_chunk(sg, lane, row, p16);
        voff = (unsigned)(row - i * kRowsPerStep) * stride + (unsigned)((p16 ^ swz(row)) * 16);
      }
      const unsigned rows = (unsigned)(tok0 + i * kRowsPerStep);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint16_t*)(Ts + sg * 512)),
          16, voff, rows * stride, 0, 0);
    }
  }
};

// 8 bf16 of row t of a u_swz tile, channels 8c .. 8c+7.
template <int D>
__device__ __forceinline__ bf16x8 lds_u_row(const uint16_t* Ts, int t, int c) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(Ts + t * D + ((c ^ u_swz<D>(t)) * 8)));
}

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
  const int off = ((c8 >> 1) ^ v_swz<D>(r)) * 8 + (c8 & 1) * 4;
  const u32x2 lo = lds_read_tr16(Vs + row * D + off);
  const u32x2 hi = lds_read_tr16(Vs + (row + 8) * D + off);
  return cat_bf16x8(lo, hi);
}

// The A operand of lds_v_operand (32 channels x rows row_base .. +15, the
// same element order) from a u_swz tile.
template <int D>
__device__ __forceinline__ bf16x8 lds_u_t_operand(const uint16_t* Ts, int lane, int dt, int row_base) {
  const int G = lane >> 4, j = lane & 15;
  const int r = j >> 2, q = j & 3;
  const int row = row_base + 4 * (G >> 1) + r;
  const int c8 = 8 * dt + 4 * (G & 1) + q;
  const int off0 = ((c8 >> 1) ^ u_swz<D>(row)) * 8 + (c8 & 1) * 4;
  const int off1 = ((c8 >> 1) ^ u_swz<D>(row + 8)) * 8 + (c8 & 1) * 4;
  const u32x2 lo = lds_read_tr16(Ts + row * D + off0);
  const u32x2 hi = lds_read_tr16(Ts + (row + 8) * D + off1);
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
