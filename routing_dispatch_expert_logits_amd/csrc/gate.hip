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
// in registers on the weight fragments as they arrive; nothing is written back.
#include "moe_kernels.h"

namespace moe {

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Exact three-way bf16 split of 8 fp32 weights: w = hi + mid + lo.
__device__ __forceinline__ void split3(f32x8 w, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  hi = __builtin_convertvector(w, bf16x8);
  const f32x8 r1 = w - __builtin_convertvector(hi, f32x8);
  mid = __builtin_convertvector(r1, bf16x8);
  lo = __builtin_convertvector(r1 - __builtin_convertvector(mid, f32x8), bf16x8);
}

// Workgroup: 4 waves as 2 (tokens) x 2 (experts); a wave owns a 64 x TN block of
// logits (TN = 32 or 64), a workgroup 128 x 2 TN.  No LDS: every lane loads its own
// MFMA operand fragments (8 consecutive k of one X row, 8 consecutive k of one Wg
// row), two 32-wide K-steps ahead of their use; the waves of a workgroup that share
// rows or experts read the same lines at about the same time, so the repeats hit
// in L1.  The kernel is bound by the rate at which a CU can have such loads in
// flight, so the wider tile (a third fewer bytes per MFMA) is faster wherever its
// K slices stay long (gate_plan).
constexpr int kGTM = 64, kGBM = 2 * kGTM;

template <int TN>
struct GateFrag {
  u32x4 a[4];            // X rows m0 + 16 fm + l % 16
  f32x4 b[TN / 16][2];   // Wg rows n0 + 16 fn + l % 16, two halves of 4 k
};

// blockIdx.y selects a K slice [y * Hs, (y + 1) * Hs), Hs a multiple of 64
// (split-K).  With one slice the result plus bias goes to logits; with several,
// slice y writes its fp32 partial to logits + y * T * E and k_gate_reduce adds
// the slices in a fixed order.
template <int TN>
__global__ __launch_bounds__(256) void k_gate(const uint16_t* __restrict__ X,
                                              const float* __restrict__ Wg,
                                              const float* __restrict__ bias,
                                              float* __restrict__ logits, int T, int E, int H,
                                              int Hs) {
  constexpr int kGFN = TN / 16, kGBN = 2 * TN;
  const int NT = ceil_div(E, kGBN);
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so workgroup
  // b runs on XCD b % 8; giving each XCD a contiguous run of (token block, expert
  // block) pairs keeps the NT workgroups that read one token block on one XCD and
  // its rows in that XCD's L2 (dealt in plain order, every token block is fetched
  // into several XCDs' L2s from HBM)
  const int total = ceil_div(T, kGBM) * NT;
  const int per_xcd = ceil_div(total, 8);
  const int L = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || L >= total) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = (L / NT) * kGBM + (wave >> 1) * kGTM;
  const int n0 = (L % NT) * kGBN + (wave & 1) * TN;
  if (m0 >= T || n0 >= E) return;  // no barriers or LDS: a wave with no logits leaves
  const int kbeg = blockIdx.y * Hs;
  if (gridDim.y > 1) {
    logits += (size_t)blockIdx.y * T * E;
    bias = nullptr;
  }
  const int kl = (lane >> 4) * 8;
  const uint16_t* pa[4];
  const float* pb[kGFN];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) pa[fm] = X + (size_t)min(m0 + fm * 16 + (lane & 15), T - 1) * H + kbeg + kl;
#pragma unroll
  for (int fn = 0; fn < kGFN; ++fn) pb[fn] = Wg + (size_t)min(n0 + fn * 16 + (lane & 15), E - 1) * H + kbeg + kl;

  auto load = [&](GateFrag<TN>& f, int k) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) f.a[fm] = *reinterpret_cast<const u32x4*>(pa[fm] + k);
#pragma unroll
    for (int fn = 0; fn < kGFN; ++fn) {
      f.b[fn][0] = *reinterpret_cast<const f32x4*>(pb[fn] + k);
      f.b[fn][1] = *reinterpret_cast<const f32x4*>(pb[fn] + k + 4);
    }
  };
  f32x4 acc[3][4][kGFN];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < kGFN; ++fn) acc[j][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const GateFrag<TN>& f) {
    bf16x8 bh[kGFN], bm[kGFN], bl[kGFN];
#pragma unroll
    for (int fn = 0; fn < kGFN; ++fn) {
      const f32x8 w = {f.b[fn][0][0], f.b[fn][0][1], f.b[fn][0][2], f.b[fn][0][3],
                       f.b[fn][1][0], f.b[fn][1][1], f.b[fn][1][2], f.b[fn][1][3]};
      split3(w, bh[fn], bm[fn], bl[fn]);
    }
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const bf16x8 a = as_bf16x8(f.a[fm]);
#pragma unroll
      for (int fn = 0; fn < kGFN; ++fn) {
        acc[0][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[fn], acc[0][fm][fn], 0, 0, 0);
        acc[1][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[fn], acc[1][fm][fn], 0, 0, 0);
        acc[2][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[fn], acc[2][fm][fn], 0, 0, 0);
      }
    }
  };
  // two K-steps in flight; past the end of the slice the loads repeat its last
  // step (in bounds, never consumed)
  GateFrag<TN> f0, f1;
  load(f0, 0);
  load(f1, 32);
  for (int k = 0; k < Hs; k += 64) {
    step(f0);
    load(f0, min(k + 64, Hs - 32));
    step(f1);
    load(f1, min(k + 96, Hs - 32));
  }
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < kGFN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + fm * 16 + (lane >> 4) * 4 + i;
        const int c = n0 + fn * 16 + (lane & 15);
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

GatePlan gate_plan(int T, int E, int H) {
  // split K until about 1024 waves run (each K slice a multiple of 64; a 2048-wave
  // target measured slower on the Qwen3-, DeepSeek-R1-shaped and latent layers);
  // the 64-wide tile when its slices stay at least 1024 long (measured: 18 % faster
  // on the DeepSeek-R1-shaped and latent gates, 6 % slower on the Qwen3-shaped one,
  // whose 128 experts would need 8 slices of 256)
  auto splits = [&](int tn) {
    const int waves = ceil_div(T, kGBM) * ceil_div(E, 2 * tn) * 4;
    int s = 1;
    while (waves * s < 1024 && s < 8 && H % (64 * s * 2) == 0) s *= 2;
    return s;
  };
  const int s64 = splits(64);
  if (H / s64 >= 1024) return GatePlan{64, s64};
  return GatePlan{32, splits(32)};
}

hipError_t launch_gate_bf16(const uint16_t* x, const float* gate_w, const float* bias, float* logits,
                            float* partial, int T, int E, int H, hipStream_t st, bool defer_reduce,
                            int* splits) {
  const GatePlan p = gate_plan(T, E, H);
  const int S = p.splits;
  if (splits) *splits = S;
  const int Hs = H / S;
  const dim3 g(ceil_div(ceil_div(T, kGBM) * ceil_div(E, 2 * p.tn), 8) * 8, S), b(256);
  float* dst = S > 1 ? partial : logits;
  if (p.tn == 64)
    hipLaunchKernelGGL(k_gate<64>, g, b, 0, st, x, gate_w, bias, dst, T, E, H, Hs);
  else
    hipLaunchKernelGGL(k_gate<32>, g, b, 0, st, x, gate_w, bias, dst, T, E, H, Hs);
  if (S > 1 && !defer_reduce) {  // deferred: the top-k kernel sums the slices as it reads them
    const size_t n = (size_t)T * E;
    hipLaunchKernelGGL(k_gate_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, partial, S,
                       bias, logits, T, E);
  }
  return hipGetLastError();
}

}  // namespace moe
