// Combine: unpermute the expert outputs and apply the routing weights (step a6).
//
// The combine reverses the route and the source unpermutes and applies the
// routing weights (WideEP explainer (Kimi K3), "The router writes a network
// schedule"); it moves about the same volume as the dispatch ("Top-k
// multiplies traffic. Locality subtracts it.").
//
// out[t] = sum_j w[t,j] * Y[token_row[t,j]] (+ add[t]) with one fp32 fma per
// term in ascending j, the optional addend (a shared expert's output, which
// every token receives with weight 1) added last, and one rounding to the output
// type.  The fused kernel gathers the k rows directly; the unfused pair first
// unpermutes into token order and then reduces, with the same fma sequence, so
// both give the same bits.  An assignment dropped by an expert capacity
// (token_row = -1) contributes no term; the kept weights are used as they are.
#include "moe_kernels.h"

namespace moe {

template <typename IT>
struct Vec16;  // 16 bytes of input elements
template <>
struct Vec16<uint16_t> {
  static constexpr int n = 8;
  __device__ static void unpack(uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  __device__ static void unpack(uint4 v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

template <int N>
__device__ __forceinline__ void store_out(void* out, size_t elem0, const float* acc, bool f32) {
  if (f32) {
    float* o = static_cast<float*>(out) + elem0;
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4*>(o + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + elem0;
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
    if constexpr (N == 8) {
      *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
    }
  }
}

// acc[i] += the addend's 16-byte chunk, element by element in fp32
template <typename IT>
__device__ __forceinline__ void add_row(float* acc, uint4 v) {
  float f[Vec16<IT>::n];
  Vec16<IT>::unpack(v, f);
#pragma unroll
  for (int i = 0; i < Vec16<IT>::n; ++i) acc[i] += f[i];
}

constexpr int kCombTokPerWg = 4;  // one wave per token

// Expert outputs are read exactly once: a nontemporal load streams them past the caches
// instead of evicting what other kernels keep there.  Measured on the R1-shaped combine
// (940 MB of rows): 218 -> 192 us, the same bits.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Fused: one wave per token, each lane owns 16-byte column chunks of the row.
// A pass covers CH chunks per lane (c, c + 64, ...), so CH * 1 KB of each row, and
// gathers U of the k rows at once: U * CH 16-byte loads per lane are in flight
// together.  The launcher takes CH large enough that one or two passes cover the
// row: measured on 8192 x 7168 and 4096 x 2048 combines (8 of 256 / 128 experts,
// rows in expert order), reading each row in one piece rather than in 2 KB pieces
// took 4096 x 2048 from 37 to 29.6 us and 8192 x 7168 from 195 to 190 us, with the
// same bits.  TOK: the rows are the unpermuted ones, token t's j-th at t * k + j (the
// second step of the unfused pair), still skipped where token_row[t, j] = -1.
template <typename IT, int U, int CH, bool TOK>
__global__ __launch_bounds__(256) void k_combine(const uint4* __restrict__ y, int row16,
                                                 const int32_t* __restrict__ token_row,
                                                 const float* __restrict__ topk_w,
                                                 const uint4* __restrict__ add, int T, int k,
                                                 void* __restrict__ out, int out_f32) {
  constexpr int NV = Vec16<IT>::n;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kCombTokPerWg + (threadIdx.x >> 6);
  if (t >= T) return;
  const int c0 = (int)((long)row16 * blockIdx.y / gridDim.y);
  const int c1 = (int)((long)row16 * (blockIdx.y + 1) / gridDim.y);
  int my_row = 0;
  float my_w = 0.f;
  if (lane < k) {
    my_row = token_row[(size_t)t * k + lane];
    if (TOK && my_row >= 0) my_row = t * k + lane;
    my_w = topk_w[(size_t)t * k + lane];
  }
  // The trip counts are wave-uniform so every lane takes part in the shuffles of
  // the row indices and weights (a shuffle from an inactive lane returns no
  // defined value); lanes past the end of the row clamp their loads and store
  // nothing, and rows past the k-th are neither loaded nor summed.
  for (int cb = c0; cb < c1; cb += CH * kWave) {
    bool on[CH];
    int c[CH];
    float acc[CH][NV];
#pragma unroll
    for (int h = 0; h < CH; ++h) {
      on[h] = cb + h * kWave + lane < c1;
      c[h] = on[h] ? cb + h * kWave + lane : c1 - 1;
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[h][i] = 0.f;
    }
    for (int j = 0; j < k; j += U) {
      uint4 v[U][CH];
      float wj[U];
      int r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        r[u] = __shfl(my_row, (j + u) & (kWave - 1), kWave);
        wj[u] = __shfl(my_w, (j + u) & (kWave - 1), kWave);
        if (j + u >= k) r[u] = -1;
        const uint4* yr = y + (size_t)max(r[u], 0) * row16;
#pragma unroll
        for (int h = 0; h < CH; ++h)
          v[u][h] = r[u] >= 0 ? load_stream(yr + c[h]) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r[u] < 0) continue;  // dropped, or past the k-th row (uniform over the wave)
#pragma unroll
        for (int h = 0; h < CH; ++h) {
          float f[NV];
          Vec16<IT>::unpack(v[u][h], f);
#pragma unroll
          for (int i = 0; i < NV; ++i) acc[h][i] = fmaf(wj[u], f[i], acc[h][i]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < CH; ++h) {
      if (!on[h]) continue;
      if (add) add_row<IT>(acc[h], add[(size_t)t * row16 + c[h]]);
      store_out<NV>(out, ((size_t)t * row16 + c[h]) * NV, acc[h], out_f32 != 0);
    }
  }
}

// Unfused step 1: y_tok[t*k + j] = Y[token_row[t, j]] (one wave per assignment);
// dropped assignments (-1) are skipped.  Also the plain row gather
// dst[a] = src[index[a]] for a < min(R, *limit) (limit nullable).
__global__ __launch_bounds__(256) void k_unpermute(const uint4* __restrict__ y, int row16,
                                                   const int32_t* __restrict__ token_row, int R,
                                                   const int32_t* __restrict__ limit,
                                                   uint4* __restrict__ y_tok) {
  const int lane = threadIdx.x & 63;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (a >= R || (limit && a >= *limit)) return;
  const int r = token_row[a];
  if (r < 0) return;
  const uint4* src = y + (size_t)r * row16;
  uint4* dst = y_tok + (size_t)a * row16;
  for (int c = lane; c < row16; c += kWave) store_stream(dst + c, load_stream(src + c));
}

// tok: the rows are y_tok[t * k + j] (unfused step 2), else y[token_row[t, j]]
static hipError_t launch_combine_rows(const void* y, int row16, bool in_bf16, const int32_t* token_row,
                                     const float* w, const void* add, int T, int k, void* out,
                                     bool out_f32, bool tok, hipStream_t st) {
  // split columns until ~1024 workgroups (small token counts)
  const int gx = ceil_div(T, kCombTokPerWg);
  int cs = 1;
  while (gx * cs < 1024 && row16 / (cs * 2) >= kWave) cs *= 2;
  const dim3 g(gx, cs), b(256);
  // chunks per lane and pass: enough for one or two passes over a workgroup's
  // columns (at most 8), with U * CH = 16 loads in flight per lane
  const int width = ceil_div(row16, cs);
  int ch = 1;
  while (ch < 8 && ch * kWave < width) ch *= 2;
#define MOE_COMB(IT, U, CH)                                                                     \
  if (tok)                                                                                      \
    hipLaunchKernelGGL((k_combine<IT, U, CH, true>), g, b, 0, st, static_cast<const uint4*>(y), \
                       row16, token_row, w, static_cast<const uint4*>(add), T, k, out,          \
                       (int)out_f32);                                                           \
  else                                                                                          \
    hipLaunchKernelGGL((k_combine<IT, U, CH, false>), g, b, 0, st, static_cast<const uint4*>(y), \
                       row16, token_row, w, static_cast<const uint4*>(add), T, k, out,          \
                       (int)out_f32)
#define MOE_COMB_CH(IT)                       \
  if (ch == 1) { MOE_COMB(IT, 8, 1); }        \
  else if (ch == 2) { MOE_COMB(IT, 8, 2); }   \
  else if (ch == 4) { MOE_COMB(IT, 4, 4); }   \
  else { MOE_COMB(IT, 2, 8); }
  if (in_bf16) {
    MOE_COMB_CH(uint16_t)
  } else {
    MOE_COMB_CH(float)
  }
#undef MOE_COMB_CH
#undef MOE_COMB
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, int row16, bool in_bf16, const int32_t* token_row,
                          const float* w, const void* add, int T, int k, void* out, bool out_f32,
                          hipStream_t st) {
  return launch_combine_rows(y, row16, in_bf16, token_row, w, add, T, k, out, out_f32, false, st);
}

hipError_t launch_unpermute(const void* y, int row16, const int32_t* token_row, int R,
                            const int32_t* limit, void* y_tok, hipStream_t st) {
  hipLaunchKernelGGL(k_unpermute, dim3(ceil_div(R, 4)), dim3(256), 0, st,
                     static_cast<const uint4*>(y), row16, token_row, R, limit,
                     static_cast<uint4*>(y_tok));
  return hipGetLastError();
}

// Unfused step 2: out[t] = sum_j w[t, j] * y_tok[t*k + j] (dropped terms skipped), the
// fused kernel's fma order over the unpermuted rows, so the same bits.
hipError_t launch_weighted_reduce(const void* y_tok, int row16, bool in_bf16, const int32_t* token_row,
                                  const float* w, const void* add, int T, int k, void* out,
                                  bool out_f32, hipStream_t st) {
  return launch_combine_rows(y_tok, row16, in_bf16, token_row, w, add, T, k, out, out_f32, true, st);
}

}  // namespace moe
