// fg_quant.hip -- fp32 -> OCP E4M3 block quantisers producing the operands of
// the block-scaled GEMM: one fp32 scale per 1x128 block of an activation and
// per 128x128 block of a weight, scale = amax / 448, values divided by the
// scale, clamped to [-448, 448] and rounded to nearest E4M3 with ties to even.
//
// Sources: the 2kiu.com DeepGEMM explainer, section 4.4 (scale factors derived
// from the data's statistics; out-of-range values clipped/saturated) and the
// zwzgs.cn DeepGEMM page, "Features > fine-grained scaling". The 1x128 and
// 128x128 granularity, amax/448 and round-to-nearest-even are the readings
// taken where the pages stop.
//
// The _pow2 entry points round each scale up to a power of two (at least
// 2^-126), the E8M0 block scales of the MX / micro-scaling formats the 2kiu.com
// explainer points to in section 7; dividing by such a scale is exact.
//
// Inputs must be finite. Both kernels are bandwidth-bound streaming passes:
// each input byte is read once, each code byte written once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fg.h"
#include "fg_e4m3.hpp"

namespace {

using fg::block_scale;
using fg::pow2_up;

// Four codes of a block with scale s (pow2: s is a power of two and the
// division is a multiplication by its exact reciprocal).
__device__ __forceinline__ uint32_t encode4(float4 v, float s, int pow2) {
  return pow2 ? fg::e4m3x4_mul(v.x, v.y, v.z, v.w, 1.0f / s) : fg::e4m3x4_div(v.x, v.y, v.z, v.w, s);
}

__device__ __forceinline__ float amax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// 1x128 blocks: 32 lanes per block (4 floats each), 8 blocks per 256-thread
// workgroup. x [batch][M][K] -> q [batch][M][K], sa [batch][K/128][M].
__global__ __launch_bounds__(256) void quant_act_1x128(const float* __restrict__ x,
                                                       uint8_t* __restrict__ q,
                                                       float* __restrict__ sa,
                                                       int M, int K, long blocks, int pow2) {
  const long blk = (long)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (blk >= blocks) return;
  const int l = threadIdx.x & 31;
  const int KB = K / 128;
  const long row = blk / KB;          // global row over batch*M
  const int kb = (int)(blk - row * KB);
  const long off = row * K + (long)kb * 128 + l * 4;
  const float4 v = *(const float4*)(x + off);
  float m = amax4(v);
#pragma unroll
  for (int d = 16; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 32));
  float s = block_scale(m);
  if (pow2) s = pow2_up(s);
  *(uint32_t*)(q + off) = encode4(v, s, pow2);
  if (l == 0) {
    const long b = row / M, r = row - b * M;
    sa[(b * KB + kb) * (long)M + r] = s;
  }
}

// 128x128 blocks: one 256-thread workgroup per block, 16 float4 per thread.
// w [G][N][K] -> q [G][N][K], sb [G][ceil(N/128)][K/128]. When N is not a
// multiple of 128 the last row block of each expert holds the remaining
// N mod 128 rows: its amax (and so its scale) comes from those rows alone, and
// nothing past row N is read or written.
__global__ __launch_bounds__(256) void quant_weight_128x128(const float* __restrict__ w,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ sb, int N, int K, int pow2) {
  __shared__ float red[4];
  const int KB = K / 128;
  const int NB = (N + 127) / 128;
  const long blk = blockIdx.x;
  const long gnb = blk / KB;          // (expert, row block) pair
  const int kb = (int)(blk - gnb * KB);
  const long g = gnb / NB;
  const int nb = (int)(gnb - g * NB);
  const int t = threadIdx.x;
  const int col = (t & 31) * 4;       // 32 threads cover one 128-wide row
  const int r0 = nb * 128 + (t >> 5); // 8 rows per pass, 16 passes
  const float* wg = w + g * (long)N * K;
  uint8_t* qg = q + g * (long)N * K;
  float4 v[16];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = r0 + i * 8;
    v[i] = row < N ? *(const float4*)(wg + (long)row * K + (long)kb * 128 + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    m = fmaxf(m, amax4(v[i]));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = block_scale(m);
  if (pow2) s = pow2_up(s);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = r0 + i * 8;
    if (row < N) *(uint32_t*)(qg + (long)row * K + (long)kb * 128 + col) = encode4(v[i], s, pow2);
  }
  if (t == 0) sb[gnb * KB + kb] = s;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int quant_act(const float* x, void* q, float* sa, int batch, int M, int K, hipStream_t stream, int pow2) {
  if (batch < 0 || M < 0 || K < 128 || K % 128) return FG_EINVAL;
  if (batch == 0 || M == 0) return FG_OK;
  if (!x || !q || !sa || !aligned(x, 16) || !aligned(q, 4) || !aligned(sa, 4)) return FG_EINVAL;
  const long blocks = (long)batch * M * (K / 128);
  const long grid = (blocks + 7) / 8;
  if (grid > 0x7fffffffL) return FG_EINVAL;
  hipLaunchKernelGGL(quant_act_1x128, dim3((unsigned)grid), dim3(256), 0, stream, x,
                     static_cast<uint8_t*>(q), sa, M, K, blocks, pow2);
  return hipGetLastError() == hipSuccess ? FG_OK : FG_ELAUNCH;
}

int quant_weight(const float* w, void* q, float* sb, int G, int N, int K, hipStream_t stream, int pow2) {
  if (G < 0 || N < 0 || K < 128 || K % 128) return FG_EINVAL;
  if (G == 0 || N == 0) return FG_OK;
  if (!w || !q || !sb || !aligned(w, 16) || !aligned(q, 4) || !aligned(sb, 4)) return FG_EINVAL;
  const long grid = (long)G * ((N + 127) / 128) * (K / 128);
  if (grid > 0x7fffffffL) return FG_EINVAL;
  hipLaunchKernelGGL(quant_weight_128x128, dim3((unsigned)grid), dim3(256), 0, stream, w,
                     static_cast<uint8_t*>(q), sb, N, K, pow2);
  return hipGetLastError() == hipSuccess ? FG_OK : FG_ELAUNCH;
}

}  // namespace

extern "C" {

// Declared in fg.h.
int fg_quant_act_1x128(const float* x, void* q, float* sa, int batch, int M, int K,
                       hipStream_t stream) {
  return quant_act(x, q, sa, batch, M, K, stream, 0);
}

int fg_quant_weight_128x128(const float* w, void* q, float* sb, int G, int N, int K,
                            hipStream_t stream) {
  return quant_weight(w, q, sb, G, N, K, stream, 0);
}

int fg_quant_act_1x128_pow2(const float* x, void* q, float* sa, int batch, int M, int K,
                            hipStream_t stream) {
  return quant_act(x, q, sa, batch, M, K, stream, 1);
}

int fg_quant_weight_128x128_pow2(const float* w, void* q, float* sb, int G, int N, int K,
                                 hipStream_t stream) {
  return quant_weight(w, q, sb, G, N, K, stream, 1);
}

}  // extern "C"
