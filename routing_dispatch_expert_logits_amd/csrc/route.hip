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

// One workgroup per 64-token ranking block: 16 waves x 4 tokens.  Each wave
// holds one token's E scores as 64-bit keys (order_key(score) << 32 | ~expert),
// so a plain max picks the larger score and, on equal scores, the lower expert
// index.  k rounds of wave-max extract the top k in order.  Counts per expert
// for the block are gathered in LDS (order-independent) and written to
// block_counts[block][e].
template <int SLOTS>
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ scores_in,
                                               const float* __restrict__ bias, int T, int E, int k,
                                               int32_t* __restrict__ topk_ids,
                                               float* __restrict__ topk_w,
                                               int32_t* __restrict__ block_counts) {
  __shared__ int cnt[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();

  for (int i = 0; i < 4; ++i) {
    const int t = blockIdx.x * kBlockTok + wave * 4 + i;
    if (t >= T) break;
    const float* row = scores_in + (size_t)t * E;
    uint64_t key[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int e = lane + s * kWave;
      if (e < E) {
        float v = row[e];
        if (bias) v = v + bias[e];
        key[s] = (static_cast<uint64_t>(order_key(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
      } else {
        key[s] = 0;  // below every real key
      }
    }
    int my_e = 0;
    float my_s = 0.f, top = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int s = 1; s < SLOTS; ++s) best = key[s] > best ? key[s] : best;
      best = wave_max_u64(best);
      const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
      const float sc = key_to_score(static_cast<uint32_t>(best >> 32));
      if (j == 0) top = sc;
      if (lane == j) { my_e = e; my_s = sc; }
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        if (lane + s * kWave == e) key[s] = 0;
    }
    // Renormalised softmax over the selected k: the full-E denominator cancels.
    const float ex = lane < k ? expf(my_s - top) : 0.f;
    const float sum = wave_sum_f32(ex);
    if (lane < k) {
      topk_ids[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = ex / sum;
      atomicAdd(&cnt[my_e], 1);
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
  const int t0 = blockIdx.x * kBlockTok;
  const int n = min(kBlockTok, T - t0) * k;
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
//   bm > 0: mtile_start[e] = sum_{e' < e} ceil(count_e' / bm), mtile_start[E] = total.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ block_counts, int nb, int E,
                                               const int32_t* __restrict__ offsets_in,
                                               int32_t* __restrict__ counts_out,
                                               int32_t* __restrict__ offsets_out, int bm,
                                               int32_t* __restrict__ mtile_start) {
  __shared__ int smem[48];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int b = 0; b < nb; ++b) c += block_counts[(size_t)b * E + e];
  int total = 0;
  int off = block_exclusive_scan(e < E ? c : 0, &total, smem);
  if (offsets_in && e < E) off = offsets_in[e];
  if (e < E) {
    if (counts_out) counts_out[e] = c;
    if (offsets_out) {
      offsets_out[e] = off;
      if (e == E - 1) offsets_out[E] = off + c;
    }
    int run = off;
    for (int b = 0; b < nb; ++b) {
      const size_t i = (size_t)b * E + e;
      const int v = block_counts[i];
      block_counts[i] = run;
      run += v;
    }
  }
  if (bm > 0) {
    const int mt = e < E ? ceil_div(c, bm) : 0;
    int tot = 0;
    const int st = block_exclusive_scan(mt, &tot, smem);
    if (e < E) mtile_start[e] = st;
    if (e == E - 1) mtile_start[E] = st + mt;
  }
}

// m-tile table from given offsets (moe_grouped_ffn on its own).
__global__ __launch_bounds__(1024) void k_mtiles(const int32_t* __restrict__ offsets, int E, int bm,
                                                 int32_t* __restrict__ mtile_start) {
  __shared__ int smem[48];
  const int e = threadIdx.x;
  const int mt = e < E ? ceil_div(offsets[e + 1] - offsets[e], bm) : 0;
  int tot = 0;
  const int st = block_exclusive_scan(mt, &tot, smem);
  if (e < E) mtile_start[e] = st;
  if (e == E - 1) mtile_start[E] = st + mt;
}

// ------------------------------------------------------------------ launchers

hipError_t launch_topk(const float* scores, const float* bias, int T, int E, int k, int32_t* ids,
                       float* w, int32_t* block_counts, hipStream_t st) {
  const int nb = ceil_div(T, kBlockTok);
  const int slots = ceil_div(E, kWave);
  dim3 g(nb), b(1024);
  if (slots <= 1) hipLaunchKernelGGL(k_topk<1>, g, b, 0, st, scores, bias, T, E, k, ids, w, block_counts);
  else if (slots <= 2) hipLaunchKernelGGL(k_topk<2>, g, b, 0, st, scores, bias, T, E, k, ids, w, block_counts);
  else if (slots <= 4) hipLaunchKernelGGL(k_topk<4>, g, b, 0, st, scores, bias, T, E, k, ids, w, block_counts);
  else if (slots <= 8) hipLaunchKernelGGL(k_topk<8>, g, b, 0, st, scores, bias, T, E, k, ids, w, block_counts);
  else hipLaunchKernelGGL(k_topk<16>, g, b, 0, st, scores, bias, T, E, k, ids, w, block_counts);
  return hipGetLastError();
}

hipError_t launch_block_counts(const int32_t* ids, int T, int E, int k, int32_t* block_counts,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_block_counts, dim3(ceil_div(T, kBlockTok)), dim3(256), 0, st, ids, T, E, k,
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
