// Top-k expert selection, routing weights, per-block expert counts and the
// count/offset scan (steps a2-a3 of the routed-expert layer).
//
// The source rank turns gating scores into k expert ids per token and the
// dispatcher counts assignments per destination and allocates each expert a
// contiguous slot range (WideEP explainer (Kimi K3), "The router writes a
// network schedule"; k distinct experts per token, "Sparse compute. Dense
// availability.").  Counts are assignments, not unique tokens ("Three
// Parameter Counts...", "What the utilization dashboard smooths away").
//
// Everything stays on the device: counts feed the offsets, the offsets feed the
// permutation and the grouped GEMM's tile table, and the host never reads them.
#include "moe_kernels.h"

namespace moe {

// One workgroup per ranking block of 16 * tpw tokens: 16 waves x tpw tokens
// (tpw = 4 for 64-token blocks, 1 for 16-token blocks).  A wave holds
// one token's E scores as order keys (order_key(score): larger score, larger
// key).  Each of the k rounds takes the wave-wide largest key, then the lowest
// expert index holding it (so equal scores go to the lower index), and removes
// that entry; both reductions are DPP row butterflies plus readlane.  Counts per
// expert for the block are gathered in LDS (order-independent) and written to
// block_counts[block][e].
template <int SLOTS, int G>
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ scores_in,
                                               const float* __restrict__ bias, int T, int E, int k,
                                               int32_t* __restrict__ topk_ids,
                                               float* __restrict__ topk_w,
                                               int32_t* __restrict__ block_counts) {
  __shared__ int cnt[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();

  // the scores of G tokens (G <= tokens per wave) are loaded before their
  // selection work starts
  const int tpw = block_tokens(T) / 16;
  float bv[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = lane + s * kWave;
    bv[s] = (bias && e < E) ? bias[e] : 0.f;
  }
  for (int g0 = 0; g0 < tpw; g0 += G) {
    const int tbase = blockIdx.x * 16 * tpw + wave * tpw + g0;
    float sv[G][SLOTS];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int t = min(tbase + i, T - 1);
      const float* row = scores_in + (size_t)t * E;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int e = lane + s * kWave;
        sv[i][s] = e < E ? row[e] : 0.f;
      }
    }
    // The G tokens run through the k rounds together: their wave reductions are
    // independent, so their latencies overlap.  Tokens past the end (clamped
    // rows above) are ranked too but write nothing.
    uint32_t key[G][SLOTS];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int e = lane + s * kWave;
        const float v = bias ? sv[i][s] + bv[s] : sv[i][s];
        key[i][s] = e < E ? order_key(v) : 0u;  // 0 is below every real key
      }
    int my_e[G];
    float my_s[G], top[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      my_e[i] = 0;
      my_s[i] = 0.f;
      top[i] = 0.f;
    }
    for (int j = 0; j < k; ++j) {
      uint32_t best[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        uint32_t lm = key[i][0];
#pragma unroll
        for (int s = 1; s < SLOTS; ++s) lm = max(lm, key[i][s]);
        best[i] = wave_max_u32(lm);
      }
      int sel[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        uint32_t li = 0xffffffffu;
#pragma unroll
        for (int s = SLOTS - 1; s >= 0; --s)
          if (key[i][s] == best[i]) li = static_cast<uint32_t>(lane + s * kWave);
        sel[i] = static_cast<int>(wave_min_u32(li));
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float sc = key_to_score(best[i]);
        if (j == 0) top[i] = sc;
        if (lane == j) {
          my_e[i] = sel[i];
          my_s[i] = sc;
        }
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
          if (lane + s * kWave == sel[i]) key[i][s] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int t = tbase + i;
      // Renormalised softmax over the selected k: the full-E denominator cancels.
      const float ex = lane < k ? expf(my_s[i] - top[i]) : 0.f;
      const float sum = wave_sum_f32(ex);
      if (t < T && g0 + i < tpw && lane < k) {
        topk_ids[(size_t)t * k + lane] = my_e[i];
        topk_w[(size_t)t * k + lane] = ex / sum;
        atomicAdd(&cnt[my_e[i]], 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Per-block expert counts from given ids (moe_dispatch_permute on its own).
__global__ __launch_bounds__(256) void k_block_counts(const int32_t* __restrict__ topk_ids, int T,
                                                      int E, int k,
                                                      int32_t* __restrict__ block_counts) {
  __shared__ int cnt[kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int bt = block_tokens(T);
  const int t0 = blockIdx.x * bt;
  const int n = min(bt, T - t0) * k;
  for (int a = tid; a < n; a += 256) atomicAdd(&cnt[topk_ids[(size_t)t0 * k + a]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan over up to 1024 values, one per thread of a 1024-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* smem16) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int incl = wave_inclusive_scan(v, lane);
  if (lane == 63) smem16[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? smem16[lane] : 0;
    const int wi = wave_inclusive_scan(w, lane);
    if (lane < 16) smem16[16 + lane] = wi - w;
    if (lane == 15) smem16[32] = wi;
  }
  __syncthreads();
  const int res = smem16[16 + wave] + incl - v;
  *total = smem16[32];
  __syncthreads();
  return res;
}

// Counts -> offsets -> per-block row bases (+ the GEMM m-tile table).
//   block_counts[b][e] in: assignments of expert e in ranking block b;
//                      out: first row of block b's assignments to e.
//   offsets_in  non-NULL: use these segment starts (moe_dispatch_permute);
//               NULL: write counts_out / offsets_out from the block counts.
//   bm > 0: GEMM m-tile tables for two tile heights, bm and 2 bm:
//           mtile_start[e] = sum_{e' < e} ceil(count_e' / bm), mtile_start[E] = total,
//           and the same for 2 bm at mtile_start[E + 1 + e].
// Thread t works on expert t % E and on the P = 1024 / E contiguous block ranges
// of part t / E, so the column sums and the per-block prefix run P-wide.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ block_counts, int nb, int E,
                                               const int32_t* __restrict__ offsets_in,
                                               int32_t* __restrict__ counts_out,
                                               int32_t* __restrict__ offsets_out, int bm,
                                               int32_t* __restrict__ mtile_start) {
  __shared__ int smem[48];
  __shared__ int psum[1024];
  __shared__ int off_s[kMaxE];
  const int t = threadIdx.x;
  const int P = 1024 / E;
  const int e = t % E, p = t / E;
  const bool active = p < P;
  const int b0 = active ? (int)((long)nb * p / P) : 0;
  const int b1 = active ? (int)((long)nb * (p + 1) / P) : 0;
  // loads are batched eight at a time so their latencies overlap
  constexpr int U = 8;
  int part = 0;
  {
    int b = b0;
    for (; b + U <= b1; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = block_counts[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) part += v[u];
    }
    for (; b < b1; ++b) part += block_counts[(size_t)b * E + e];
  }
  if (active) psum[p * E + e] = part;
  __syncthreads();
  int c = 0;
  if (t < E)
    for (int q = 0; q < P; ++q) c += psum[q * E + t];
  int total = 0;
  int off = block_exclusive_scan(t < E ? c : 0, &total, smem);
  if (t < E) {
    if (offsets_in) off = offsets_in[t];
    off_s[t] = off;
    if (counts_out) counts_out[t] = c;
    if (offsets_out) {
      offsets_out[t] = off;
      if (t == E - 1) offsets_out[E] = off + c;
    }
  }
  __syncthreads();
  if (active) {
    int run = off_s[e];
    for (int q = 0; q < p; ++q) run += psum[q * E + e];
    int b = b0;
    for (; b + U <= b1; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = block_counts[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        block_counts[(size_t)(b + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; b < b1; ++b) {
      const size_t i = (size_t)b * E + e;
      const int v = block_counts[i];
      block_counts[i] = run;
      run += v;
    }
  }
  if (bm > 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mt = t < E ? ceil_div(c, bm << h) : 0;
      int tot = 0;
      const int st = block_exclusive_scan(mt, &tot, smem);
      int32_t* tab = mtile_start + h * (E + 1);
      if (t < E) tab[t] = st;
      if (t == E - 1) tab[E] = st + mt;
    }
  }
}

// m-tile tables (tile heights bm and 2 bm, as in k_scan) from given offsets
// (moe_grouped_ffn on its own).
__global__ __launch_bounds__(1024) void k_mtiles(const int32_t* __restrict__ offsets, int E, int bm,
                                                 int32_t* __restrict__ mtile_start) {
  __shared__ int smem[48];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int mt = e < E ? ceil_div(c, bm << h) : 0;
    int tot = 0;
    const int st = block_exclusive_scan(mt, &tot, smem);
    int32_t* tab = mtile_start + h * (E + 1);
    if (e < E) tab[e] = st;
    if (e == E - 1) tab[E] = st + mt;
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_topk(const float* scores, const float* bias, int T, int E, int k, int32_t* ids,
                       float* w, int32_t* block_counts, hipStream_t st) {
  const int nb = ceil_div(T, block_tokens(T));
  const int slots = ceil_div(E, kWave);
  const bool one = block_tokens(T) == 16;  // one token per wave
  dim3 g(nb), b(1024);
#define MOE_TOPK(SL, GG) \
  hipLaunchKernelGGL((k_topk<SL, GG>), g, b, 0, st, scores, bias, T, E, k, ids, w, block_counts)
  if (one) {
    if (slots <= 1) MOE_TOPK(1, 1);
    else if (slots <= 2) MOE_TOPK(2, 1);
    else if (slots <= 4) MOE_TOPK(4, 1);
    else if (slots <= 8) MOE_TOPK(8, 1);
    else MOE_TOPK(16, 1);
  } else {
    if (slots <= 1) MOE_TOPK(1, 4);
    else if (slots <= 2) MOE_TOPK(2, 4);
    else if (slots <= 4) MOE_TOPK(4, 4);
    else if (slots <= 8) MOE_TOPK(8, 4);
    else MOE_TOPK(16, 2);
  }
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_block_counts(const int32_t* ids, int T, int E, int k, int32_t* block_counts,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_block_counts, dim3(ceil_div(T, block_tokens(T))), dim3(256), 0, st, ids, T, E, k,
                     block_counts);
  return hipGetLastError();
}

hipError_t launch_scan(int32_t* block_counts, int nb, int E, const int32_t* offsets_in,
                       int32_t* counts_out, int32_t* offsets_out, int bm, int32_t* mtile_start,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, block_counts, nb, E, offsets_in,
                     counts_out, offsets_out, bm, mtile_start);
  return hipGetLastError();
}

hipError_t launch_mtiles(const int32_t* offsets, int E, int bm, int32_t* mtile_start,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_mtiles, dim3(1), dim3(1024), 0, st, offsets, E, bm, mtile_start);
  return hipGetLastError();
}

}  // namespace moe
