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
// token in two 64-bit masks per expert).
constexpr int kSmallT = 128;
// Largest ceil(T / 16) * k * ceil(E / 64) (ranking work per wave) for which the
// decode-scale routing runs in one workgroup; above it, over ceil(T / kMultiTok)
// workgroups that rank kMultiTok tokens each.
constexpr int kSmallRankWork = 640;
constexpr int kMultiTok = 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (NaN stays NaN), by gfx950's bf16 conversion
// instruction: one instruction and no temporaries, which keeps the GEMM epilogues
// inside the register budget of three waves per SIMD.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// 8 bf16 values of one 16-byte chunk, widened exactly to fp32.
__device__ __forceinline__ void unpack_bf16x8(uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
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

__host__ __device__ __forceinline__ bool route_one_workgroup(int T, int E, int k) {
  return ceil_div(T, kBlockTok) * k * ceil_div(E, kWave) <= kSmallRankWork;
}

// ---- MXFP8 (OCP MX: E4M3 elements, one E8M0 scale per 32 elements along K)

constexpr int kMxBlock = 32;

// E8M0 scale code of a block whose largest magnitude is amax (finite, >= 0):
// 127 + floor(log2 amax) - 8, clamped at 0 (fp32 zeros and subnormals land there).
__device__ __forceinline__ int mx_scale_code(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);  // biased exponent
  return e == 0 ? 0 : max(e - 8, 0);
}

// 2^-(code - 127) as an fp32 multiplier (code 0..246 gives a normal number).
__device__ __forceinline__ float mx_inv_scale(int code) {
  return __uint_as_float(static_cast<uint32_t>(254 - code) << 23);
}

// Four E4M3 codes (bytes 0..3 = a, b, c, d) of values already divided by the block
// scale: clamped to +-448 first (the conversion rounds to nearest even but turns
// magnitudes from 464 on into NaN), then converted by the hardware.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, 0, false)) & 0xffffu;
  return lo | (hi << 16);
}

// MX-quantise 8 consecutive values of a 32-element block held by 4 adjacent lanes
// (lanes 4j .. 4j+3 hold the block's elements 0-7, 8-15, 16-23, 24-31).  Every lane
// of the group must be active.  Returns the 8 codes; *code = the block's E8M0 scale.
__device__ __forceinline__ uint2 mx_quantize8(const float* f, int* code) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  m = fmaxf(m, __shfl_xor(m, 2, kWave));
  const int c = mx_scale_code(m);
  const float inv = mx_inv_scale(c);
  *code = c;
  return make_uint2(e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                    e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
}

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
