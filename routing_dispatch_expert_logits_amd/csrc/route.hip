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

// A pointer every lane of the wave holds, moved to scalar registers (the caller
// guarantees it is wave-uniform), so loads through it take a scalar base.
template <class P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<P*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Between accesses of one wave to its own LDS slice: the LDS serves a wave's
// instructions in issue order, so only the compiler must keep them in order.
__device__ __forceinline__ void lds_order() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Top-k of one wave's keys (SLOTS per lane, entry lane + 64 s, expert index
// < E real) by a threshold.  Each lane's largest key belongs to a different
// entry, so if at least k lane maxima reach tau, the k-th largest key reaches it
// too and every entry of the top k has a key >= tau.  tau is the largest value
// with zero low 16 bits for which that holds (a bitwise search over the lane
// maxima).  The real entries with key >= tau (typically k to 1.5 k of them) are
// packed into one per lane through the wave's 64-entry LDS slice, and each takes
// its exact position in the order from a pass over the others; the first k are
// the top k, since every other entry's key is below tau.  Returns false, with
// nothing written, when more than 64 entries reach tau (heavy ties); the caller
// then ranks in rounds.  On success lane j < k holds the j-th expert and its
// score (from the key, so -0.0 reads back as +0.0, as in the rounds).
template <int SLOTS>
__device__ __forceinline__ bool rank_by_threshold(const uint32_t (&key)[SLOTS], int E, int k, int lane,
                                                  uint32_t* __restrict__ lkey, int* __restrict__ lidx,
                                                  int& my_e, float& my_s) {
  uint32_t lm = key[0];
#pragma unroll
  for (int s = 1; s < SLOTS; ++s) lm = max(lm, key[s]);
  uint32_t tau = 0;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t c = tau | (1u << b);
    if (__popcll(__ballot(lm >= c)) >= k) tau = c;
  }
  // the candidates' masks are formed twice (count, then place) rather than kept:
  // SLOTS 64-bit masks held across both loops spilled at 16 slots
  int n = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) n += __popcll(__ballot(lane + s * kWave < E && key[s] >= tau));
  if (n > kWave) return false;
  int base = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const bool in = lane + s * kWave < E && key[s] >= tau;
    const unsigned long long m = __ballot(in);
    if (in) {
      const int at = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
      lkey[at] = key[s];
      lidx[at] = lane + s * kWave;
    }
    base += __popcll(m);
  }
  lds_order();
  const uint32_t ck = lane < n ? lkey[lane] : 0u;
  const int ci = lane < n ? lidx[lane] : 0x7fffffff;
  int pos = 0;
  for (int j = 0; j < n; ++j) {
    const uint32_t kj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ck), j));
    const int ij = __builtin_amdgcn_readlane(ci, j);
    pos += (kj > ck || (kj == ck && ij < ci)) ? 1 : 0;
  }
  lds_order();
  if (lane < n && pos < k) {
    lkey[pos] = ck;
    lidx[pos] = ci;
  }
  lds_order();
  my_e = lane < k ? lidx[lane] : 0;
  my_s = lane < k ? key_to_score(lkey[lane]) : 0.f;
  lds_order();  // read before the slice's next use
  return true;
}

// The k experts of one token, ranked by one wave: lane j < k receives the j-th
// expert id and its renormalised weight.  Scores become order keys
// (order_key(score): larger score, larger key), and the order is larger key
// first, then the lower expert index (so equal scores go to the lower index).
// Two exact ways to the same k: rank_by_threshold below, and, where its candidate
// set is too large, k rounds that each take the wave-wide largest key, then the
// lowest expert index holding it, and remove that entry (both reductions DPP row
// butterflies plus readlane).
// The token's scores come from src (see ScoreSrc): a scores row plus an optional
// bias formed on the fly, or the gate's split-K partial rows summed in ascending
// slice order plus the bias, the sum then written out as the token's logits row
// (the arithmetic of k_gate_reduce, so the logits are the same bits).
// lkey / lidx: the wave's 64-entry LDS slice for rank_by_threshold.
template <int SLOTS>
__device__ __forceinline__ void rank_token(const ScoreSrc& src, size_t row0, int E, int k, int lane,
                                           uint32_t* lkey, int* lidx, int& my_e, float& my_w) {
  // every load is issued unconditionally (lanes past E read the last score and
  // are masked afterwards) so they overlap instead of each waiting in a branch.
  // The row is the same for the whole wave: a scalar base plus 32-bit lane offsets
  // (per-slot 64-bit addresses overflowed the register budget at 16 slots).
  float v[SLOTS];
  const float* first = uniform_ptr((src.parts ? src.parts : src.scores) + row0);
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) v[s] = first[static_cast<unsigned>(min(lane + s * kWave, E - 1))];
  for (int p = 1; p < src.S; ++p) {
    float q[SLOTS];
    const float* part = uniform_ptr(src.parts + (size_t)p * src.stride + row0);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) q[s] = part[static_cast<unsigned>(min(lane + s * kWave, E - 1))];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) v[s] += q[s];
  }
  if (src.bias) {
    float b[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) b[s] = src.bias[static_cast<unsigned>(min(lane + s * kWave, E - 1))];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) v[s] += b[s];
  }
  if (src.logits_out) {
    float* lrow = uniform_ptr(src.logits_out + row0);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (lane + s * kWave < E) lrow[static_cast<unsigned>(lane + s * kWave)] = v[s];
  }
  uint32_t key[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s)
    key[s] = lane + s * kWave < E ? order_key(v[s]) : 0u;  // 0 is below every real key
  my_e = 0;
  float my_s = 0.f, top = 0.f;
  // the threshold pass costs about as much as the rounds below at 2 slots and far
  // less from 4 on (E = 896, k = 16: about 500 instead of 1900 instructions)
  if (SLOTS >= 4 && rank_by_threshold<SLOTS>(key, E, k, lane, lkey, lidx, my_e, my_s)) {
    top = __shfl(my_s, 0, kWave);
  } else {
  for (int j = 0; j < k; ++j) {
    uint32_t lm = key[0];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s) lm = max(lm, key[s]);
    const uint32_t best = wave_max_u32(lm);
    uint32_t li = 0xffffffffu;
#pragma unroll
    for (int s = SLOTS - 1; s >= 0; --s)
      if (key[s] == best) li = static_cast<uint32_t>(lane + s * kWave);
    const int e = static_cast<int>(wave_min_u32(li));
    const float sc = key_to_score(best);
    if (j == 0) top = sc;
    if (lane == j) {
      my_e = e;
      my_s = sc;
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (lane + s * kWave == e) key[s] = 0u;
  }
  }
  // Renormalised softmax over the selected k: the full-E denominator cancels.
  const float ex = lane < k ? expf(my_s - top) : 0.f;
  const float sum = wave_sum_f32(ex);
  my_w = ex / sum;
}

// One workgroup per 16-token ranking block, one token per wave.  Counts per
// expert for the block are gathered in LDS (order-independent) and written to
// block_counts[block][e].
template <int SLOTS>
__global__ __launch_bounds__(1024) void k_topk(ScoreSrc src, int T, int E, int k,
                                               int32_t* __restrict__ topk_ids,
                                               float* __restrict__ topk_w,
                                               int32_t* __restrict__ block_counts) {
  static_assert(kBlockTok == 16, "one token per wave of a 1024-thread workgroup");
  __shared__ int cnt[kMaxE];
  __shared__ uint32_t rk_key[16][kWave];
  __shared__ int rk_idx[16][kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();

  const int t = blockIdx.x * kBlockTok + wave;
  if (t < T) {
    int my_e;
    float my_w;
    rank_token<SLOTS>(src, (size_t)t * E, E, k, lane, rk_key[wave], rk_idx[wave], my_e, my_w);
    if (lane < k) {
      topk_ids[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = my_w;
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

// Per-expert scan of the block counts: block_counts[b][e] (rows of expert e in
// ranking block b) becomes the number of rows of e in the blocks before b, and
// counts_out[e] (if non-NULL) the expert's total, or min(total, cap) with an
// expert capacity cap > 0 (the slots allocated; later assignments are dropped).  Workgroup x covers experts
// 64x .. 64x + 63, one per lane, so every load is a coalesced 256-byte row slice;
// its 16 waves split the blocks into 16 contiguous ranges.  The experts'
// segment starts are added by the consumer (offsets[e] + base), so no
// workgroup waits for another.
__global__ __launch_bounds__(1024) void k_expert_scan(int32_t* __restrict__ block_counts, int nb,
                                                      int E, int cap,
                                                      int32_t* __restrict__ counts_out) {
  __shared__ int psum[16][kWave];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * kWave + lane;
  const bool on = e < E;
  const int b0 = (int)((long)nb * w / 16), b1 = (int)((long)nb * (w + 1) / 16);
  constexpr int U = 16;  // loads in flight per lane
  int part = 0;
  if (on) {
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
  psum[w][lane] = part;
  __syncthreads();
  int run = 0, total = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int v = psum[q][lane];
    run += q < w ? v : 0;
    total += v;
  }
  if (on && w == 0 && counts_out) counts_out[e] = cap > 0 ? min(total, cap) : total;
  if (on) {
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
}

// Segment starts and GEMM m-tile tables from the per-expert counts (or, when
// offsets_in is given, from those segment starts).
//   offsets_out non-NULL: offsets_out[e] = sum_{e' < e} counts[e'], offsets_out[E] = total.
//   bm > 0: m-tile tables for two tile heights, bm and 2 bm:
//           mtile_start[e] = sum_{e' < e} ceil(count_e' / bm), mtile_start[E] = total,
//           and the same for 2 bm at mtile_start[E + 1 + e].
__global__ __launch_bounds__(1024) void k_offsets(const int32_t* __restrict__ counts,
                                                  const int32_t* __restrict__ offsets_in, int E,
                                                  int32_t* __restrict__ offsets_out, int bm,
                                                  int32_t* __restrict__ mtile_start) {
  __shared__ int smem[48];
  const int t = threadIdx.x;
  const int c = t < E ? (offsets_in ? offsets_in[t + 1] - offsets_in[t] : counts[t]) : 0;
  if (offsets_out) {
    int total = 0;
    const int off = block_exclusive_scan(c, &total, smem);
    if (t < E) offsets_out[t] = off;
    if (t == E - 1) offsets_out[E] = off + c;
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
    if (t < kClaimSlots) mtile_start[2 * (E + 1) + t] = 0;
  }
}

// Decode-scale routing (T <= 64 MW, MW = 1 or 2): top-k per token (one wave per
// token), counts, offsets, the GEMM m-tile tables and the row metadata in one
// launch, for what the large-T path does in three.  Row order inside an expert's
// segment is ascending token id, as there: row = offsets[e] + (number of lower
// tokens in mask[e]), mask[e] the tokens that picked e (MW 64-bit words, built with
// order-independent LDS atomicOr).  With an expert capacity cap > 0, assignments
// ranked cap or later in their expert are dropped (token_row = -1) and counts are
// min(count, cap).
template <int MW>
struct RouteLds {
  int cnt[kMaxE];
  int off_s[kMaxE];
  unsigned long long mask[kMaxE * MW];
  int ids[64 * MW * kWave];  // [t][j], t < T, j < k
  int smem[48];
  uint32_t rk_key[16][kWave];
  int rk_idx[16][kWave];
};

template <int MW>
__device__ __forceinline__ void route_clear(RouteLds<MW>& L, int E) {
  for (int e = threadIdx.x; e < E; e += 1024) {
    L.cnt[e] = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) L.mask[e * MW + w] = 0ull;
  }
}

// One assignment of token t: its count and its bit in the expert's token mask.
template <int MW>
__device__ __forceinline__ void route_note(RouteLds<MW>& L, int t, int j, int k, int e) {
  L.ids[t * k + j] = e;
  atomicAdd(&L.cnt[e], 1);
  atomicOr(&L.mask[e * MW + (t >> 6)], 1ull << (t & 63));
}

// Counts, offsets, m-tile tables and row metadata from the noted assignments
// (all T * k of them in L, after a barrier).
template <int MW>
__device__ __forceinline__ void route_metadata(RouteLds<MW>& L, int T, int E, int k,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ row_token, int32_t* __restrict__ token_row,
                                               int cap, int bm, int32_t* __restrict__ mtile_start) {
  const int tid = threadIdx.x;
  const int c = tid < E ? (cap > 0 ? min(L.cnt[tid], cap) : L.cnt[tid]) : 0;
  int total = 0;
  const int off = block_exclusive_scan(c, &total, L.smem);
  if (tid < E) {
    L.off_s[tid] = off;
    counts[tid] = c;
    offsets[tid] = off;
    if (tid == E - 1) offsets[E] = off + c;
  }
  if (bm > 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mt = tid < E ? ceil_div(c, bm << h) : 0;
      int tot = 0;
      const int st = block_exclusive_scan(mt, &tot, L.smem);
      int32_t* tab = mtile_start + h * (E + 1);
      if (tid < E) tab[tid] = st;
      if (tid == E - 1) tab[E] = st + mt;
    }
    if (tid < kClaimSlots) mtile_start[2 * (E + 1) + tid] = 0;
  }
  __syncthreads();
  for (int a = tid; a < T * k; a += 1024) {
    const int t = a / k, e = L.ids[a];
    int rank = __popcll(L.mask[e * MW + (t >> 6)] & ((1ull << (t & 63)) - 1ull));
#pragma unroll
    for (int w = 0; w + 1 < MW; ++w)
      if (w < (t >> 6)) rank += __popcll(L.mask[e * MW + w]);
    if (cap > 0 && rank >= cap) {
      token_row[a] = -1;  // dropped: past the expert's capacity
    } else {
      token_row[a] = L.off_s[e] + rank;
      row_token[L.off_s[e] + rank] = t;
    }
  }
}

// In one workgroup: every wave ranks tokens wave, wave + 16, ... one after another.
template <int SLOTS, int MW>
__global__ __launch_bounds__(1024) void k_route_small(
    ScoreSrc src, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ token_row,
    int cap, int bm, int32_t* __restrict__ mtile_start) {
  __shared__ RouteLds<MW> L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  route_clear(L, E);
  __syncthreads();
  for (int t = wave; t < T; t += 16) {
    int my_e;
    float my_w;
    rank_token<SLOTS>(src, (size_t)t * E, E, k, lane, L.rk_key[wave], L.rk_idx[wave], my_e, my_w);
    if (lane < k) {
      topk_ids[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = my_w;
      route_note(L, t, lane, k, my_e);
    }
  }
  __syncthreads();
  route_metadata(L, T, E, k, counts, offsets, row_token, token_row, cap, bm, mtile_start);
}

// Over ceil(T / 4) workgroups, one token per wave in the first 4 waves (one ranking
// wave per SIMD: 16 ranking waves on one CU's four SIMDs took twice as long), for
// steps whose ranking is too much work for one CU; all 16 waves of the workgroup that
// writes the metadata take part in it.  No workgroup waits for another.  Each writes its tokens'
// ids and weights and then counts itself in a hand-over word (release): the word
// holds this call's tag (a value no earlier call used) above an 8-bit count, and a
// word with any other tag, whatever an earlier call or the workspace left there,
// counts as zero.  The atomic that brings the count to the number of workgroups is
// exactly one, and its workgroup (acquire) sees every id: it writes the counts,
// offsets, tile tables and row metadata and clears the word (a replayed graph repeats
// its tag).  Installing the tag is a compare-and-swap, which fails only when another
// workgroup's succeeded in between; after that every count is a plain atomic add.
template <int SLOTS, int MW>
__global__ __launch_bounds__(1024) void k_route_multi(
    ScoreSrc src, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ token_row,
    int cap, int bm, int32_t* __restrict__ mtile_start, unsigned long long* __restrict__ handover,
    unsigned long long tag) {
  __shared__ RouteLds<MW> L;
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kMultiTok + wave;
  if (wave < kMultiTok && t < T) {
    int my_e;
    float my_w;
    rank_token<SLOTS>(src, (size_t)t * E, E, k, lane, L.rk_key[wave], L.rk_idx[wave], my_e, my_w);
    if (lane < k) {
      topk_ids[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = my_w;
    }
    // the waves that wrote release their writes (each release writes back the L2)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // Count this workgroup: the first to arrive swaps the tag in (a stale word, from
    // any other call, counts as zero), the others add 1 (no retries among them; the
    // word keeps the tag until the metadata writer clears it, after every count).
    unsigned long long old = __hip_atomic_load(handover, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long cnt;
    for (;;) {
      if ((old >> 8) == tag) {
        cnt = (__hip_atomic_fetch_add(handover, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) & 0xffu) + 1;
        break;
      }
      if (__hip_atomic_compare_exchange_strong(handover, &old, (tag << 8) | 1ull, __ATOMIC_ACQ_REL,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        cnt = 1;
        break;
      }
    }
    s_last = (int)cnt == (int)gridDim.x;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) __hip_atomic_store(handover, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  route_clear(L, E);
  __syncthreads();
  for (int a = threadIdx.x; a < T * k; a += 1024) route_note(L, a / k, a % k, k, topk_ids[a]);
  __syncthreads();
  route_metadata(L, T, E, k, counts, offsets, row_token, token_row, cap, bm, mtile_start);
}

// One group of T rows (the shared expert's GEMMs run as a single expert).
__global__ void k_single_group(int T, int32_t* __restrict__ offsets, int bm,
                               int32_t* __restrict__ mtile_start) {
  if (threadIdx.x < kClaimSlots) mtile_start[4 + threadIdx.x] = 0;
  if (threadIdx.x != 0) return;
  offsets[0] = 0;
  offsets[1] = T;
  mtile_start[0] = 0;
  mtile_start[1] = ceil_div(T, bm);
  mtile_start[2] = 0;
  mtile_start[3] = ceil_div(T, 2 * bm);
}

// ------------------------------------------------------------------ launchers

hipError_t launch_topk(const ScoreSrc& src, int T, int E, int k, int32_t* ids, float* w,
                       int32_t* block_counts, hipStream_t st) {
  const int nb = ceil_div(T, block_tokens(T));
  const int slots = ceil_div(E, kWave);
  dim3 g(nb), b(1024);
  if (slots <= 1) hipLaunchKernelGGL(k_topk<1>, g, b, 0, st, src, T, E, k, ids, w, block_counts);
  else if (slots <= 2) hipLaunchKernelGGL(k_topk<2>, g, b, 0, st, src, T, E, k, ids, w, block_counts);
  else if (slots <= 4) hipLaunchKernelGGL(k_topk<4>, g, b, 0, st, src, T, E, k, ids, w, block_counts);
  else if (slots <= 8) hipLaunchKernelGGL(k_topk<8>, g, b, 0, st, src, T, E, k, ids, w, block_counts);
  else hipLaunchKernelGGL(k_topk<16>, g, b, 0, st, src, T, E, k, ids, w, block_counts);
  return hipGetLastError();
}

hipError_t launch_block_counts(const int32_t* ids, int T, int E, int k, int32_t* block_counts,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_block_counts, dim3(ceil_div(T, block_tokens(T))), dim3(256), 0, st, ids, T, E, k,
                     block_counts);
  return hipGetLastError();
}

hipError_t launch_expert_scan(int32_t* block_counts, int nb, int E, int cap, int32_t* counts_out,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_expert_scan, dim3(ceil_div(E, kWave)), dim3(1024), 0, st, block_counts, nb, E,
                     cap, counts_out);
  return hipGetLastError();
}

hipError_t launch_offsets(const int32_t* counts, const int32_t* offsets_in, int E,
                          int32_t* offsets_out, int bm, int32_t* mtile_start, hipStream_t st) {
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, st, counts, offsets_in, E, offsets_out, bm,
                     mtile_start);
  return hipGetLastError();
}

hipError_t launch_route_small(const ScoreSrc& src, int T, int E, int k, int32_t* ids,
                             float* w, int32_t* counts, int32_t* offsets, int32_t* row_token,
                             int32_t* token_row, int cap, int bm, int32_t* mtile_start,
                             unsigned long long* handover, unsigned long long tag, hipStream_t st) {
  // the tag sits above an 8-bit count of at most ceil(128 / 4) workgroups
  if (T > kSmallT || tag == 0 || (tag >> 56) != 0) return hipErrorInvalidValue;
  const int slots = ceil_div(E, kWave);
  const bool one = route_one_workgroup(T, E, k);
  if (!one && !handover) return hipErrorInvalidValue;
  const dim3 b(1024);
#define MOE_RS(SL, MW)                                                                              \
  if (one)                                                                                          \
    hipLaunchKernelGGL((k_route_small<SL, MW>), dim3(1), b, 0, st, src, T, E, k, ids, w, counts,    \
                       offsets, row_token, token_row, cap, bm, mtile_start);                        \
  else                                                                                              \
    hipLaunchKernelGGL((k_route_multi<SL, MW>), dim3(ceil_div(T, kMultiTok)), b, 0, st, src, T, E, \
                       k, ids, w, counts, offsets, row_token, token_row, cap, bm, mtile_start,      \
                       handover, tag)
#define MOE_RS_SLOTS(MW)          \
  if (slots <= 1) { MOE_RS(1, MW); } \
  else if (slots <= 2) { MOE_RS(2, MW); } \
  else if (slots <= 4) { MOE_RS(4, MW); } \
  else if (slots <= 8) { MOE_RS(8, MW); } \
  else { MOE_RS(16, MW); }
  if (T <= 64) {
    MOE_RS_SLOTS(1)
  } else {
    MOE_RS_SLOTS(2)
  }
#undef MOE_RS_SLOTS
#undef MOE_RS
  return hipGetLastError();
}

hipError_t launch_single_group(int T, int32_t* offsets, int bm, int32_t* mtile_start, hipStream_t st) {
  hipLaunchKernelGGL(k_single_group, dim3(1), dim3(64), 0, st, T, offsets, bm, mtile_start);
  return hipGetLastError();
}

}  // namespace moe
