// MXFP8 conversion kernel: rows of bf16 or fp32 values -> E4M3 codes + one E8M0
// scale per 32 consecutive elements of a row (the conversion kernel and scale
// metadata of a low-precision dispatch: WideEP explainer, "Top-k multiplies
// traffic. Locality subtracts it.").  The scale of a block with largest magnitude
// m is 2^(floor(log2 m) - 8), each element is divided by it (exactly: a power of
// two), clamped to +-448 and rounded to the nearest E4M3 value, ties to even.
#include "moe_kernels.h"

namespace moe {

// One lane per 8 consecutive elements of the flattened [rows x cols] array (cols a
// multiple of 32, so a block never straddles rows and the 4 lanes of a block are
// adjacent lanes of one wave).  n8 = rows * cols / 8 is a multiple of 4, so a block's
// lanes are all in range or all out of range.
template <typename ST>
__global__ __launch_bounds__(256) void k_mx_quantize(const ST* __restrict__ src, long n8,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float f[8];
  if constexpr (sizeof(ST) == 2) {
    unpack_bf16x8(reinterpret_cast<const uint4*>(src)[i], f);
  } else {
    const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  int code;
  const uint2 c8 = mx_quantize8(f, &code);
  reinterpret_cast<uint2*>(q)[i] = c8;
  if ((i & 3) == 0) scale[i >> 2] = static_cast<uint8_t>(code);
}

hipError_t launch_mx_quantize(const void* src, bool src_bf16, long rows, long cols, uint8_t* q,
                              uint8_t* scale, hipStream_t st) {
  if (cols % kMxBlock) return hipErrorInvalidValue;
  const long n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 g((unsigned)((n8 + 255) / 256)), b(256);
  if (src_bf16)
    hipLaunchKernelGGL(k_mx_quantize<uint16_t>, g, b, 0, st, static_cast<const uint16_t*>(src), n8, q, scale);
  else
    hipLaunchKernelGGL(k_mx_quantize<float>, g, b, 0, st, static_cast<const float*>(src), n8, q, scale);
  return hipGetLastError();
}

}  // namespace moe
