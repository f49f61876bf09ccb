// fg_kernel.hpp -- gfx950 kernel for the FP8 (OCP E4M3) block-scaled GEMM
// D = A . B^T with per-1x128 (A) and per-128x128 (B) fp32 scales and
// two-level FP32 accumulation, in the dense, MoE-contiguous and MoE-masked
// layouts.
//
// Method: the zwzgs.cn page "DeepGEMM: an open-source FP8 GEMM library",
// "Technical details > two-level accumulation": the matrix-core FP8 partial
// sums are accumulated a second time in FP32 on the general-purpose ALUs.
// Here every 128-wide K-block is one v_mfma_f32_16x16x128_f8f6f4 per 16x16
// sub-tile with a zero C operand (a fresh FP32 partial covering exactly one
// scale block), followed by one v_fma_f32 per output element that adds
// partial * (sa * sb) into the master accumulator held in VGPRs.
//
// Operand roles. The MFMA's first operand is fed with rows of B (output
// columns n), its second with rows of A (output rows m). The 16x16 result then
// gives each lane four consecutive n for a single m, so a lane needs one
// activation scale per sub-tile row and its four results form one 8-byte bf16
// store.
//
// K order inside a fragment. The hardware sums a 128-long dot product; which
// lane/byte holds which k does not change the sum as long as both operands use
// the same placement. Lane l (row l % 16, quarter q = l / 16) holds bytes
// [16q, 16q+16) and [64+16q, 64+16q+16) of its row's K-block, i.e. two 16-byte
// LDS reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

typedef int   i32x4 __attribute__((ext_vector_type(4)));
typedef int   i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };

constexpr int kKBlock = 128;   // scale block along K (elements == bytes)
constexpr int kThreads = 256;  // 4 waves of 64

struct Params {
  const uint8_t* A;       // E4M3 [rows][K] (masked: [G][M][K])
  const float* sa;        // [K/128][rows] (masked: [G][K/128][M])
  const uint8_t* B;       // E4M3 [N][K] (grouped: [G][N][K])
  const float* sb;        // [N/128][K/128] (grouped: [G][N/128][K/128])
  uint16_t* D;            // bf16 bits [rows][N] (masked: [G][M][N])
  const int32_t* m_indices;  // contiguous: expert per row, -1 = padding
  const int32_t* masked_m;   // masked: valid rows per expert
  int M;                  // rows (dense/contiguous) or M_max (masked)
  int N, K, G;
  int KB;                 // K / 128
  int tiles_m, tiles_n;   // tile grid of one group
};

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 16-byte chunk c (0..7) of tile row r lives at chunk c ^ (r & 7): the eight
// rows a quarter-wave reads for one chunk index land in eight different
// 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kKBlock + ((chunk ^ (row & 7)) << 4);
}

template <int LAYOUT, int BM, int BN>
__global__ __launch_bounds__(kThreads) void fp8_bs_gemm(Params p) {
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile must split into 2x2 waves of 16-row sub-tiles");
  constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
  constexpr int TM = WM / 16, TN = WN / 16; // 16x16 sub-tiles per wave
  constexpr int LA = BM * 8 / kThreads;     // 16-byte A chunks per thread per K-block
  constexpr int LB = BN * 8 / kThreads;
  static_assert(LA >= 1 && LB >= 1, "tile too small for the loader");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * kKBlock];
  __shared__ int s_group;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lq = lane >> 4;

  // ---- tile -> (group, m-block, n-block)
  int tile = blockIdx.x;
  int g = 0;
  if (LAYOUT == kMasked) {
    const int per = p.tiles_m * p.tiles_n;
    g = tile / per;
    tile -= g * per;
  }
  const int mb = tile / p.tiles_n;
  const int nbk = tile - mb * p.tiles_n;
  const int m0 = mb * BM, n0 = nbk * BN;

  int rows_valid = p.M;  // rows of this slab that have an output
  if (LAYOUT == kMasked) {
    int mm = p.masked_m[g];
    mm = mm < 0 ? 0 : (mm > p.M ? p.M : mm);
    if (m0 >= mm) return;  // uniform over the workgroup
    rows_valid = mm;
  }
  if (LAYOUT == kContiguous) {
    if (t == 0) s_group = -1;
    __syncthreads();
    if (t < BM && m0 + t < p.M) {
      const int id = p.m_indices[m0 + t];
      if (id >= 0 && id < p.G) atomicMax(&s_group, id);
    }
    __syncthreads();
    g = s_group;
    if (g < 0) return;  // all-padding block
  }

  const size_t K = (size_t)p.K;
  const int KB = p.KB;
  const uint8_t* Ag = p.A + (LAYOUT == kMasked ? (size_t)g * p.M * K : 0);
  const float* sag = p.sa + (LAYOUT == kMasked ? (size_t)g * KB * p.M : 0);
  const uint8_t* Bg = p.B + (LAYOUT != kDense ? (size_t)g * p.N * K : 0);
  const float* sbg = p.sb + (LAYOUT != kDense ? (size_t)g * (p.N / 128) * KB : 0);
  uint16_t* Dg = p.D + (LAYOUT == kMasked ? (size_t)g * p.M * p.N : 0);

  // ---- global -> register staging of one K-block (rows clamped into range;
  // clamped rows are computed but never stored)
  i32x4 ra[LA], rb[LB];
  const uint8_t* a_src[LA];
  const uint8_t* b_src[LB];
  int a_dst[LA], b_dst[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int c = t + kThreads * i, row = c >> 3, col = c & 7;
    const int m = min(m0 + row, p.M - 1);
    a_src[i] = Ag + (size_t)m * K + col * 16;
    a_dst[i] = swz(row, col);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int c = t + kThreads * i, row = c >> 3, col = c & 7;
    const int n = min(n0 + row, p.N - 1);
    b_src[i] = Bg + (size_t)n * K + col * 16;
    b_dst[i] = BM * kKBlock + swz(row, col);
  }

  // scales this lane needs: one sa per sub-tile row, one sb per sub-tile column
  int sa_row[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) sa_row[i] = min(m0 + wm * WM + i * 16 + lr, p.M - 1);
  int sb_blk[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) sb_blk[j] = min((n0 + wn * WN + j * 16) >> 7, p.N / 128 - 1) * KB;

  float sa_nx[TM], sb_nx[TN];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *(const i32x4*)(a_src[i] + (size_t)kb * kKBlock);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *(const i32x4*)(b_src[i] + (size_t)kb * kKBlock);
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_nx[i] = sag[(size_t)kb * p.M + sa_row[i]];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb_nx[j] = sbg[sb_blk[j] + kb];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(i32x4*)(&lds[buf][a_dst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(i32x4*)(&lds[buf][b_dst[i]]) = rb[i];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  float sa_cur[TM], sb_cur[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) sa_cur[i] = sa_nx[i];
#pragma unroll
  for (int j = 0; j < TN; ++j) sb_cur[j] = sb_nx[j];
  lstore(0);
  __syncthreads();

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < KB; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < KB;
    if (more) gload(kb + 1);

    i32x8 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + i * 16 + lr;
      const i32x4 lo = *(const i32x4*)(&lds[cur][swz(row, lq)]);
      const i32x4 hi = *(const i32x4*)(&lds[cur][swz(row, lq + 4)]);
      fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WN + j * 16 + lr;
      const i32x4 lo = *(const i32x4*)(&lds[cur][BM * kKBlock + swz(row, lq)]);
      const i32x4 hi = *(const i32x4*)(&lds[cur][BM * kKBlock + swz(row, lq + 4)]);
      fb[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // fresh FP32 partial of this K-block (C = 0), format 0 = E4M3 for both
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fb[j], fa[i], zero, 0, 0, 0, 0, 0, 0);
        const float s = sa_cur[i] * sb_cur[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], s, acc[i][j][r]);
      }
    }

    if (more) {
      lstore(cur ^ 1);
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_cur[i] = sa_nx[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb_cur[j] = sb_nx[j];
    }
    __syncthreads();
  }

  // ---- epilogue: bf16 RNE, one 8-byte store per lane per sub-tile
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 16 + lr;
    bool ok = m < rows_valid;
    if (LAYOUT == kContiguous && ok) ok = p.m_indices[m] == g;
    if (!ok) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WN + j * 16 + 4 * lq;
      if (n >= p.N) continue;
      const uint32_t lo = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
      const uint32_t hi = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
      *(uint2*)(Dg + (size_t)m * p.N + n) = make_uint2(lo, hi);
    }
  }
}

}  // namespace fg
