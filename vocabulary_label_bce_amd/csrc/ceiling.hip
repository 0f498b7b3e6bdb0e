// MFMA-only ceiling of the device: the instruction the sweeps run (v_mfma_f32_32x32x16_bf16) issued back to back
// from registers, with no memory traffic, no LDS and no vector work, so that the rate it reaches -- and the
// shader clock the device holds while doing it -- bound what any kernel built on that instruction can reach.
#include "../../include/cutbce.h"
#include "common.h"

namespace cutbce {
namespace {

__device__ inline int lane_of() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Each wave keeps four independent accumulator tiles (an MFMA never waits for the previous one's result) and runs
// `iters` rounds of four MFMAs. Lane 0 of each wave records s_memtime (shader clock ticks) and s_memrealtime
// (the 100 MHz reference clock) before and after the loop: stamps[4 w + 0..3] = t0, t1, r0, r1.
__global__ void __launch_bounds__(1024) k_mfma_ceiling(int iters, long long* __restrict__ stamps) {
  const int lane = lane_of();
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.25f + 0.001f * (float)((lane + j) % 7));
    b[j] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + j) % 5));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float keep = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) keep += c0[q] + c1[q] + c2[q] + c3[q];
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  const long long w = (long long)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (lane == 0) {
    stamps[4 * w + 0] = t0;
    stamps[4 * w + 1] = keep == -1.f ? 0 : t1;  // the sums stay live (they are never -1: every product is > 0)
    stamps[4 * w + 2] = r0;
    stamps[4 * w + 3] = r1;
  }
}

// Mixing function of MurmurHash3 (its 32-bit finaliser): spreads a counter over all 32 bits.
__device__ inline uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// The same loop on random operands: four register sets of bf16 values uniform in [-1, 1) with random mantissas,
// one set per accumulator tile, as the sweeps' operand tiles hold. The multipliers draw more power on such values
// than on the near-constant ones of k_mfma_ceiling (the power follows the values inside each MFMA: one fixed
// random set gives the same rate as sets that change every MFMA), so the clock the device holds here is the one
// data like the sweeps' allows.
__global__ void __launch_bounds__(1024) k_mfma_ceiling_random(int iters, long long* __restrict__ stamps) {
  const int lane = lane_of();
  const uint32_t w = (uint32_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = fmix32(((w * 64u + (uint32_t)lane) * 4u + (uint32_t)s) * 8u + (uint32_t)j + 1u);
      a[s][j] = (__bf16)((float)(h & 0xffffu) * (1.f / 32768.f) - 1.f);
      b[s][j] = (__bf16)((float)(h >> 16) * (1.f / 32768.f) - 1.f);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
  }
  float keep = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) keep += c0[q] + c1[q] + c2[q] + c3[q];
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    // The sums stay live: each is bounded by 4 * 16 * iters products of magnitude below 1, never NaN.
    stamps[4 * (long long)w + 0] = t0;
    stamps[4 * (long long)w + 1] = keep != keep ? 0 : t1;
    stamps[4 * (long long)w + 2] = r0;
    stamps[4 * (long long)w + 3] = r1;
  }
}

}  // namespace
}  // namespace cutbce

extern "C" cutbce_status cutbce_mfma_ceiling(int blocks, int waves_per_block, int iters, long long* stamps,
                                             void* stream) {
  if (blocks < 1 || waves_per_block < 1 || waves_per_block > 16 || iters < 1) return CUTBCE_ERR_SHAPE;
  if (!stamps) return CUTBCE_ERR_NULL;
  if (((size_t)stamps) % 8) return CUTBCE_ERR_ALIGN;
  hipLaunchKernelGGL(cutbce::k_mfma_ceiling, dim3((unsigned)blocks), dim3((unsigned)(64 * waves_per_block)), 0,
                     (hipStream_t)stream, iters, stamps);
  return hipGetLastError() == hipSuccess ? CUTBCE_OK : CUTBCE_ERR_HIP;
}

extern "C" cutbce_status cutbce_mfma_ceiling_random(int blocks, int waves_per_block, int iters, long long* stamps,
                                                    void* stream) {
  if (blocks < 1 || waves_per_block < 1 || waves_per_block > 16 || iters < 1) return CUTBCE_ERR_SHAPE;
  if (!stamps) return CUTBCE_ERR_NULL;
  if (((size_t)stamps) % 8) return CUTBCE_ERR_ALIGN;
  hipLaunchKernelGGL(cutbce::k_mfma_ceiling_random, dim3((unsigned)blocks), dim3((unsigned)(64 * waves_per_block)),
                     0, (hipStream_t)stream, iters, stamps);
  return hipGetLastError() == hipSuccess ? CUTBCE_OK : CUTBCE_ERR_HIP;
}
