// Router gate scores (step a1) on bf16 MFMA at fp32 accuracy.
//
// The source rank scores every token against every expert with the
// replicated gating network (WideEP explainer (Kimi K3), "The router writes a
// network schedule"; research-vault claim IX2-0406: the gating network is part
// of the replicated non-expert weights).  logits = X Wg^T + bias with X bf16 and
// Wg fp32.
//
// Each fp32 weight is split exactly into three bf16 terms, w = hi + mid + lo
// (hi = RNE(w), mid = RNE(w - hi), lo = w - hi - mid; 8 + 8 + 8 significand bits
// cover fp32's 24).  Every bf16 x bf16 product is exact in fp32, so
// X Wg^T = X hi^T + X mid^T + X lo^T evaluated with three fp32-accumulating MFMA
// chains has the accuracy of an fp32 GEMM, at bf16 MFMA rate.  The split is done
// while staging the weight tile into LDS; nothing is written back.
#include "moe_kernels.h"

namespace moe {

constexpr int kGBK = 64;
constexpr int kGLD = kGBK + 8;
constexpr int kGBN = 64;

__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  lo = f32_to_bf16(r1 - bf16_to_f32(mid));
}

// blockIdx.y selects a K slice [y * Hs, (y + 1) * Hs) (split-K).  With one slice the
// result plus bias goes to logits; with several, slice y writes its fp32 partial to
// logits + y * T * E and k_gate_reduce adds the slices in a fixed order.
template <int BM>
__global__ __launch_bounds__(256, 2) void k_gate_split(const uint16_t* __restrict__ X,
                                                       const float* __restrict__ Wg,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ logits, int T, int E,
                                                       int H, int Hs) {
  constexpr int BN = kGBN, TM = BM / 2, TN = BN / 2, FM = TM / 16, FN = TN / 16;
  constexpr int A_PER = BM * 8 / 256;   // 16-byte bf16 chunks of the X tile per thread
  constexpr int B_PER = BN * 16 / 256;  // 16-byte fp32 chunks of the Wg tile per thread
  static_assert(A_PER >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kGLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[3][BN * kGLD];

  const int NT = ceil_div(E, BN);
  const int m0 = (blockIdx.x / NT) * BM, n0 = (blockIdx.x % NT) * BN;
  const int kbeg = blockIdx.y * Hs;
  X += kbeg;
  Wg += kbeg;
  if (gridDim.y > 1) {
    logits += (size_t)blockIdx.y * T * E;
    bias = nullptr;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // X tile loader: row (tid / 8) + 32 i, bf16 k-offset 8 * (tid % 8)
  const int arow = tid >> 3, ak = (tid & 7) * 8;
  uint32_t aoff[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) aoff[i] = (uint32_t)min(m0 + arow + 32 * i, T - 1);
  // Wg tile loader: row (tid / 16) + 16 i, fp32 k-offset 4 * (tid % 16)
  const int brow = tid >> 4, bk = (tid & 15) * 4;
  uint32_t boff[B_PER];
#pragma unroll
  for (int i = 0; i < B_PER; ++i) boff[i] = (uint32_t)min(n0 + brow + 16 * i, E - 1);

  f32x4 acc[3][FM][FN];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[j][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[A_PER];
  f32x4 rb[B_PER];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      ra[i] = *reinterpret_cast<const u32x4*>(X + (size_t)aoff[i] * H + k0 + ak);
#pragma unroll
    for (int i = 0; i < B_PER; ++i)
      rb[i] = *reinterpret_cast<const f32x4*>(Wg + (size_t)boff[i] * H + k0 + bk);
  };
  load(0);
  const int ar = wm * TM + (lane & 15), br = wn * TN + (lane & 15), kofs = (lane >> 4) * 8;
  for (int k0 = 0; k0 < Hs; k0 += kGBK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      *reinterpret_cast<u32x4*>(&sA[(arow + 32 * i) * kGLD + ak]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      uint16_t h[4], m[4], l[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split3(rb[i][q], h[q], m[q], l[q]);
      const int o = (brow + 16 * i) * kGLD + bk;
      *reinterpret_cast<uint2*>(&sB[0][o]) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
      *reinterpret_cast<uint2*>(&sB[1][o]) = make_uint2(m[0] | (uint32_t)m[1] << 16, m[2] | (uint32_t)m[3] << 16);
      *reinterpret_cast<uint2*>(&sB[2][o]) = make_uint2(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16);
    }
    __syncthreads();
    load(min(k0 + kGBK, Hs - kGBK));
#pragma unroll
    for (int ks = 0; ks < kGBK; ks += 32) {
      bf16x8 af[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sA[(ar + fm * 16) * kGLD + ks + kofs]));
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const bf16x8 bfr =
              as_bf16x8(*reinterpret_cast<const u32x4*>(&sB[j][(br + fn * 16) * kGLD + ks + kofs]));
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
            acc[j][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr, acc[j][fm][fn], 0, 0, 0);
        }
    }
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i;
        const int c = n0 + wn * TN + fn * 16 + (lane & 15);
        if (r < T && c < E) {
          float v = (acc[0][fm][fn][i] + acc[1][fm][fn][i]) + acc[2][fm][fn][i];
          if (bias) v += bias[c];
          logits[(size_t)r * E + c] = v;
        }
      }
}

// logits[t, e] = sum_{s < S} part[s][t][e] (+ bias[e]), summed in ascending s.
__global__ __launch_bounds__(256) void k_gate_reduce(const float* __restrict__ part, int S,
                                                     const float* __restrict__ bias,
                                                     float* __restrict__ logits, int T, int E) {
  const size_t n = (size_t)T * E;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = part[i];
  for (int s = 1; s < S; ++s) v += part[(size_t)s * n + i];
  if (bias) v += bias[i % E];
  logits[i] = v;
}

int gate_splits(int T, int E, int H) {
  const int NT = ceil_div(E, kGBN);
  const int tiles = ceil_div(T, 64) * NT;
  int s = 1;
  while (tiles * s < 1024 && s < 8 && H % (64 * s * 2) == 0) s *= 2;
  return s;
}

hipError_t launch_gate_bf16(const uint16_t* x, const float* gate_w, const float* bias, float* logits,
                            float* partial, int T, int E, int H, hipStream_t st) {
  const int NT = ceil_div(E, kGBN);
  // 64-row tiles; the K range is split until there are ~1024 workgroups (each K slice
  // a multiple of 64), so every workgroup runs a short K loop
  const int S = gate_splits(T, E, H);
  const int Hs = H / S;
  const dim3 g(ceil_div(T, 64) * NT, S), b(256);
  hipLaunchKernelGGL(k_gate_split<64>, g, b, 0, st, x, gate_w, bias, S > 1 ? partial : logits, T, E,
                     H, Hs);
  if (S > 1) {
    const size_t n = (size_t)T * E;
    hipLaunchKernelGGL(k_gate_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, partial, S,
                       bias, logits, T, E);
  }
  return hipGetLastError();
}

}  // namespace moe
