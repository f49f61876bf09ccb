// fg_ceiling.hip -- what this device sustains for the two resources the GEMM
// is bound by: the matrix-core ceiling of its inner loop (the K-loop
// arithmetic with no memory traffic at all) and the practical HBM read rate (a
// plain streaming read). A benchmark helper (libfg_ceiling.so, loaded by
// bench.py only), not part of the library.
//
// Each workgroup has 8 waves (two per SIMD, as in the GEMM's 256-row tiles);
// each wave holds 4 A and 8 B fragments of 16 rows x 128 E4M3 codes (a 64x128
// wave tile) and per "K-block" issues the 32 v_mfma_scale_f32_16x16x128_f8f6f4
// of that tile:
//   mode 0: each MFMA into a fresh partial (C = 0), promoted 3 MFMAs later by
//           4 FMAs per lane into the master accumulator -- the fp32-scale loop;
//   mode 1: each MFMA accumulating into the master accumulator with unit E8M0
//           scales -- the power-of-two loop (no vector-ALU promotion);
// on the codes in src (random codes measure the power the matrix cores draw
// on real data; all-zero codes show the clock when that power is low).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kTM = 4, kTN = 8, kSteps = kTM * kTN;
constexpr int kWordsPerWave = (kTM + kTN) * 8 * 64;   // fragments x 8 dwords x 64 lanes
constexpr int kWaveSets = 64;                          // distinct fragment sets in src

template <int MODE>
__global__ __launch_bounds__(512) void mfma_loop(const int* __restrict__ src, float* __restrict__ out, int iters,
                                                 float s) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int* w = src + ((blockIdx.x * 8 + wave) % kWaveSets) * kWordsPerWave;
  i32x8 a[kTM], b[kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[i][e] = w[(i * 8 + e) * 64 + lane];
#pragma unroll
  for (int j = 0; j < kTN; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) b[j][e] = w[((kTM + j) * 8 + e) * 64 + lane];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = zero;
  f32x4 part[4] = {zero, zero, zero, zero};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int i = u % kTM, j = u / kTM;
      if constexpr (MODE == 1) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, 127, 0, 127);
      } else {
        part[u % 4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], zero, 0, 0, 0, 0, 0, 0);
        const int v = (u + kSteps - 3) % kSteps;   // promote the MFMA issued 3 steps ago
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[v % kTM][v / kTM][r] = __builtin_fmaf(part[(u + 1) % 4][r], s, acc[v % kTM][v / kTM][r]);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the fragments stay opaque, so nothing is hoisted out of the loop
#pragma unroll
    for (int i = 0; i < kTM; ++i) asm volatile("" : "+v"(a[i]));
#pragma unroll
    for (int j = 0; j < kTN; ++j) asm volatile("" : "+v"(b[j]));
  }
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) t += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[blockIdx.x * 512 + threadIdx.x] = t;
}

// Streaming read of n 16-byte words: grid-stride, UNR nontemporal loads in
// flight per thread, folded into one value per thread so nothing is dropped.
template <int UNR>
__global__ __launch_bounds__(512) void stream_read(const i32x4* __restrict__ src, long n, int* __restrict__ out) {
  long i = (long)blockIdx.x * 512 + threadIdx.x;
  const long stride = (long)gridDim.x * 512;
  int acc = 0;
  for (; i + (UNR - 1) * stride < n; i += UNR * stride) {
    i32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += stride) {
    const i32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(long)blockIdx.x * 512 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Words of src the loop reads (int32 each) and FLOP one workgroup does per iteration.
int fgc_src_words() { return kWaveSets * kWordsPerWave; }
double fgc_flop_per_workgroup_iteration() { return 8.0 * kSteps * 2.0 * 16 * 16 * 128; }

// Launches the loop: mode 0 (C = 0 + promotion) or 1 (accumulate), grid
// workgroups of 512 threads, iters iterations; src holds fgc_src_words()
// words, out grid * 512 floats. Returns 0, or -1 for a bad argument, -3 if
// the launch failed.
int fgc_mfma_loop(const int* src, float* out, int mode, int grid, int iters, hipStream_t stream) {
  if (!src || !out || grid < 1 || iters < 1 || (mode != 0 && mode != 1)) return -1;
  if (mode == 0)
    hipLaunchKernelGGL(mfma_loop<0>, dim3(grid), dim3(512), 0, stream, src, out, iters, 0.5f);
  else
    hipLaunchKernelGGL(mfma_loop<1>, dim3(grid), dim3(512), 0, stream, src, out, iters, 0.5f);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Reads `bytes` (a positive multiple of 16) of device memory at src (16-byte
// aligned) with `grid` workgroups of 512 threads, each thread keeping
// `inflight` (4 or 8) 16-byte loads in flight; out holds grid * 512 ints.
// Returns 0, or -1 for a bad argument, -3 if the launch failed.
int fgc_stream_read(const void* src, long bytes, int* out, int grid, int inflight, hipStream_t stream) {
  if (!src || !out || grid < 1 || bytes < 16 || bytes % 16 || ((uintptr_t)src & 15)) return -1;
  if (inflight == 4)
    hipLaunchKernelGGL(stream_read<4>, dim3(grid), dim3(512), 0, stream, (const i32x4*)src, bytes / 16, out);
  else if (inflight == 8)
    hipLaunchKernelGGL(stream_read<8>, dim3(grid), dim3(512), 0, stream, (const i32x4*)src, bytes / 16, out);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
