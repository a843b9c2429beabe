// W8A8 FP8 projection (robotworld.top SparkDiffusion write-up, section 2.3:
// projections in FP8 E4M3 with a static per-output-channel weight scale and a
// dynamic per-token activation scale):
//
//   y[m, n] = s_x[m] * s_w[n] * sum_k E4M3(xq[m, k]) * E4M3(wq[n, k])   -> bf16
//
// xq [M, K] u8 (the per-token quantiser's codes), wq [N, K] u8 (one row per
// output channel), y [M, N] bf16.
//
// One workgroup (8 waves) computes a 256-token x 256-channel tile with
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit block scales, fp32
// accumulation). The product is taken transposed, W tile x X tile^T, so that
// an accumulator column is one token and its registers hold runs of 4
// consecutive output channels: the bf16 epilogue writes 8-byte pieces of a
// token's row. Wave (wm, wn) owns tokens 128*wm .. +127 and channels
// 64*wn .. +63: 2 x 4 MFMA tiles, 8 accumulators.
//
// The k loop goes in steps of 64 (one MFMA) through a 3-stage LDS ring of
// 16 KB operand tiles [256 rows][64 bytes], 16-byte chunk c of row r stored at
// c ^ ((r / 4) % 4): the 16 rows read by a 16-lane LDS cycle then cover all 64
// banks. Tiles arrive with buffer loads straight into LDS (two 1 KB segments
// per operand per wave per stage), issued two stages ahead; rows past M or N
// read as zeros (range-checked buffer).
//
// MFMA operand layout (checked on the hardware): A[i][k] at lane
// i + 32*(k/32), byte k%32 (8 registers); B[k][j] at lane j + 32*(k/32), byte
// k%32; D as for the other 32x32 MFMAs: D[i][j] at lane j + 32*((i/4)%2),
// register (i/8)*4 + i%4.
#include "sd_device.h"
#include "sd_launch.h"

namespace sd {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int i32x4g __attribute__((ext_vector_type(4)));

constexpr int kGT = 256;           // rows (tokens or channels) per operand tile
constexpr int kGK = 64;            // k bytes per stage
constexpr int kGStages = 3;
constexpr int kGTile = kGT * kGK;  // bytes per operand tile
constexpr int kGWaves = 8;

// Raw buffer resource over `bytes` bytes at p (offsets at or past `bytes`
// read as zero without a memory access).
__device__ __forceinline__ i32x4g gemm_rsrc(const void* p, unsigned bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4g r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at voff + soff into LDS at byte address
// lds + 16*lane. Written as inline assembly so that the compiler does not
// track the LDS write: it would otherwise put a wait for every load in
// flight in front of each LDS read of the other stages. The k loop waits for
// the stage it needs with an explicit s_waitcnt vmcnt(n) (vector-memory
// counts complete in issue order), and issues no other vector-memory
// access.
__device__ __forceinline__ void gemm_dma16(i32x4g rsrc, unsigned voff, unsigned soff, unsigned lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ unsigned gemm_lds_addr(const uint8_t* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

__device__ __forceinline__ int gsw(int r) { return (r >> 2) & 3; }

// 32 bytes of row `row`, k-half kh (bytes 32*kh .. +31) of an LDS tile.
__device__ __forceinline__ v8i gemm_operand(const uint8_t* tile, int row, int kh) {
  const uint8_t* base = tile + row * kGK;
  const i32x4g lo = *reinterpret_cast<const i32x4g*>(base + 16 * ((2 * kh) ^ gsw(row)));
  const i32x4g hi = *reinterpret_cast<const i32x4g*>(base + 16 * ((2 * kh + 1) ^ gsw(row)));
  v8i v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = lo[i];
    v[4 + i] = hi[i];
  }
  return v;
}

}  // namespace

__global__ __launch_bounds__(512, 1) void gemm_fp8_kernel(GemmFp8Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t sW[kGStages][kGTile];
  __shared__ __attribute__((aligned(16))) uint8_t sX[kGStages][kGTile];

  const int ntn = (int)((a.N + kGT - 1) / kGT);
  const int64_t tm = blockIdx.x / ntn;
  const int tn = (int)(blockIdx.x % ntn);
  const int64_t m0 = tm * kGT;
  const int64_t n0 = (int64_t)tn * kGT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  const int l32 = lane & 31, kh = lane >> 5;

  // operand buffers of this tile: rows past M (N) are outside the range
  const int64_t mrows = a.M - m0 < kGT ? a.M - m0 : kGT;
  const int64_t nrows = a.N - n0 < kGT ? a.N - n0 : kGT;
  const i32x4g xr = gemm_rsrc(a.xq + m0 * a.ldx, (unsigned)((mrows - 1) * a.ldx + a.K));
  const i32x4g wr = gemm_rsrc(a.wq + n0 * a.ldw, (unsigned)((nrows - 1) * a.ldw + a.K));
  // DMA segments: wave wv fills segments wv and wv + 8 (16 rows x 64 bytes
  // each) of both operand tiles; lane l -> row 16*seg + l/4, LDS slot l%4,
  // holding k chunk (l%4) ^ gsw(row)
  const int srow = lane >> 2;                       // row within the segment
  const int schunk = (lane & 3) ^ gsw(srow);        // gsw(16*seg + srow) == gsw(srow)
  const unsigned xvo = (unsigned)(srow * a.ldx + 16 * schunk);
  const unsigned wvo = (unsigned)(srow * a.ldw + 16 * schunk);
  const int nk = (int)(a.K / kGK);
  auto issue = [&](int ks) {
    const int st = ks % kGStages;
    // past the last stage: an offset beyond every range loads zeros
    const unsigned k0 = ks < nk ? (unsigned)(ks * kGK) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = wv + kGWaves * i;
      gemm_dma16(wr, wvo, k0 + (unsigned)(16 * seg * a.ldw), gemm_lds_addr(&sW[st][seg * 1024]));
      gemm_dma16(xr, xvo, k0 + (unsigned)(16 * seg * a.ldx), gemm_lds_addr(&sX[st][seg * 1024]));
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  issue(0);
  issue(1);
  for (int ks = 0; ks < nk; ++ks) {
    // this stage's loads are in (the next stage's 4 may be in flight), and
    // every wave is done with the stage that receives ks + 2
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    issue(ks + 2);
    const uint8_t* tw = sW[ks % kGStages];
    const uint8_t* tx = sX[ks % kGStages];
    v8i av[2], bv[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) av[i] = gemm_operand(tw, 64 * wn + 32 * i + l32, kh);
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = gemm_operand(tx, 128 * wm + 32 * j + l32, kh);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], bv[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane = token 32*j + l32 of the wave's block, registers = the
  // tile's channels 8*(r/4) + 4*kh + r%4
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + 128 * wm + 32 * j + l32;
    if (m >= a.M) continue;
    const float sxm = a.sx[m];
    uint16_t* yrow = a.y + m * a.ldy;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + 64 * wn + 32 * i + 8 * g + 4 * kh;
        if (n + 4 <= a.N) {
          const f32x4 s = *reinterpret_cast<const f32x4*>(a.sw + n);
          u32x2 o;
          o[0] = pack_bf16x2(acc[i][j][4 * g] * sxm * s[0], acc[i][j][4 * g + 1] * sxm * s[1]);
          o[1] = pack_bf16x2(acc[i][j][4 * g + 2] * sxm * s[2], acc[i][j][4 * g + 3] * sxm * s[3]);
          *reinterpret_cast<u32x2*>(yrow + n) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < a.N) yrow[n + e] = (uint16_t)f32_to_bf16_bits(acc[i][j][4 * g + e] * sxm * a.sw[n + e]);
        }
      }
  }
}

hipError_t launch_gemm_fp8(const GemmFp8Args& a, hipStream_t stream) {
  const int64_t tiles = ((a.M + kGT - 1) / kGT) * ((a.N + kGT - 1) / kGT);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3((unsigned)tiles), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sd
