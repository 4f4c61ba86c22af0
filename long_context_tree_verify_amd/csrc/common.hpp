// Device helpers for the gfx950 kernels: bf16 handling, wave64 reductions,
// hardware exp2/log2, the ancestor bitmask by pointer jumping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace hsv {

constexpr int kWave = 64;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kNegInf = -__builtin_huge_valf();

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// v_exp_f32 / v_log_f32: base-2 hardware transcendentals.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  uint32_t lo = __shfl(static_cast<uint32_t>(x), src, kWave);
  uint32_t hi = __shfl(static_cast<uint32_t>(x >> 32), src, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Ancestor bitmask of draft node `lane` (lanes >= n return 0).
// Pointer jumping: after round k, `anc` holds the ancestors within distance
// 2^(k+1)-1 and `jump` points 2^(k+1) levels up; six rounds cover any path in
// a 64-node tree.  `bad` is set (wave-uniform) if a parent is out of range.
__device__ __forceinline__ uint64_t tree_ancestors(const int32_t *parent_row, int n, int lane,
                                                   bool *bad) {
  int p = lane < n ? parent_row[lane] : -1;
  bool invalid = lane < n && (p < -1 || p >= lane);
  *bad = __any(invalid);
  if (invalid) p = -1;
  uint64_t anc = lane < n ? (uint64_t{1} << lane) : 0;
  int jump = p;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    uint64_t up = shfl_u64(anc, jump < 0 ? lane : jump);
    int jj = __shfl(jump, jump < 0 ? lane : jump, kWave);
    if (jump >= 0) {
      anc |= up;
      jump = jj;
    }
  }
  return anc;
}

template <int IN>
struct Elem;
template <>
struct Elem<kF32> {
  using T = float;
  __device__ static float load(const T *p, int64_t i) { return p[i]; }
};
template <>
struct Elem<kBF16> {
  using T = uint16_t;
  __device__ static float load(const T *p, int64_t i) { return bf16_to_f32(p[i]); }
};

}  // namespace hsv
