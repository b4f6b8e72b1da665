// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
// Tokens per ranking block (one bit per token in a mask): the top-k kernel ranks
// one block per workgroup, one token per wave, so T / 16 workgroups spread over
// the CUs (64-token blocks left most CUs idle at T = 4096).
constexpr int kBlockTok = 16;
__host__ __device__ __forceinline__ int block_tokens(int) { return kBlockTok; }
constexpr int kMaxE = 1024;
// Largest token count routed by the one-workgroup decode-scale kernel (one bit per
// token in a 64-bit mask).
constexpr int kSmallT = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Monotone map of an fp32 score to uint32 (larger score -> larger key); -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t o) {
  return (o & 0x80000000u) ? __uint_as_float(o & 0x7fffffffu) : __uint_as_float(~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Wave-wide unsigned max / min with DPP row operations (butterfly inside each row
// of 16 lanes: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror), then the four row results through readlane.  Every lane must be
// active.  The result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  v = min(v, dpp_u32<0x141>(v));
  v = min(v, dpp_u32<0x140>(v));
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return min(min(a, b), min(c, d));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Largest e in [0, E] with starts[e] <= q (starts non-decreasing, starts[0] = 0).
__device__ __forceinline__ int upper_index(const int32_t* __restrict__ starts, int E, int q) {
  int lo = 0, hi = E;  // invariant: starts[lo] <= q
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
