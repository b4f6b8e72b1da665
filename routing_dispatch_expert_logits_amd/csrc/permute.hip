// Permutation of token rows into expert-contiguous rows + routing metadata (step a4).
//
// The dispatcher copies token rows into buffers ordered by destination and adds
// routing metadata; the receiver groups rows by expert
// (WideEP explainer (Kimi K3), "The router writes a network schedule").  On
// one GPU the destination is the expert itself, so one permutation does both.
// The buffer holds exactly T*k*D elements: the dispatch payload T x k x H x B
// of "Top-k multiplies traffic. Locality subtracts it." with every assignment
// local and no padding.
//
// Row order inside an expert's segment is ascending token id, independent of
// scheduling: row = offsets[e] + base[block][e] + (number of lower tokens of the
// same 16-token ranking block that picked e), the latter a popcount of a per-expert
// token bitmask built with order-independent LDS atomicOr.  With an expert capacity
// cap > 0 an assignment whose rank in its expert (base + popcount) is cap or more
// is dropped: token_row = -1 and no row is written (dropping changes the model's
// output: WideEP explainer, "An imbalanced router creates a network hotspot").
#include "moe_kernels.h"

namespace moe {

constexpr int kCopyUnroll = 4;

// Exclusive prefix sum of f(i), i < n <= 1024, over the 256 threads of a workgroup
// into out[0, n) (LDS); returns the total.  Thread t takes i = 4t .. 4t + 3.
template <class F>
__device__ __forceinline__ int wg256_exclusive_scan(F f, int n, int* out, int* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[4], s = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * tid + u;
    v[u] = i < n ? f(i) : 0;
    s += v[u];
  }
  int incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = incl - s;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  const int total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * tid + u;
    if (i < n) out[i] = base;
    base += v[u];
  }
  __syncthreads();
  return total;
}

// With x_perm == NULL only the metadata is written (row_token, token_row): the
// fused layer's persistent gate/up GEMM then gathers the token rows itself.
//
// Workgroup (blockIdx.x, blockIdx.y): 4 waves x tpw tokens starting at
// blockIdx.x * 4 * tpw, columns [c0, c1) of their rows (16-byte units; the
// column split lets small token counts still fill the GPU).  Only the
// blockIdx.y == 0 workgroups write the metadata.  x / x_perm rows are row16
// 16-byte units long.
//
// MX = true (MXFP8 dispatch of bf16 rows): each token's row is quantised once (8
// elements per lane, the 4 lanes of a 32-element block adjacent) and its E4M3 codes
// (x_perm as bytes, rows of row16 * 8 codes) and E8M0 scales (xs, row16 / 4 per row)
// are copied to its destinations: the dispatch carries one byte per element plus
// one scale byte per 32.  Column splits then fall on multiples of 4 chunks.
template <bool MX>
__global__ __launch_bounds__(256) void k_permute(const u32x4* __restrict__ x, int row16,
                                                 const int32_t* __restrict__ topk_ids, int T,
                                                 int E, int k, int tpw, int cap,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ bases,
                                                 u32x4* __restrict__ x_perm,
                                                 uint8_t* __restrict__ xs,
                                                 int32_t* __restrict__ row_token,
                                                 int32_t* __restrict__ token_row,
                                                 PermuteOffsets po) {
  __shared__ unsigned long long mask[kMaxE];
  __shared__ int off_s[kMaxE];
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (po.counts) {  // segment starts from the counts (workgroup-uniform branch)
    const int32_t* cn = po.counts;
    const int tot = wg256_exclusive_scan([=](int i) { return cn[i]; }, E, off_s, wtot);
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      if (po.offsets_out) {
        for (int e = tid; e < E; e += 256) po.offsets_out[e] = off_s[e];
        if (tid == 0) po.offsets_out[E] = tot;
      }
      if (po.bm > 0) {  // m-tile tables for tile heights bm and 2 bm, claim counters cleared
        __shared__ int mt_s[kMaxE];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int bmh = po.bm << h;
          const int mtot = wg256_exclusive_scan([=](int i) { return ceil_div(cn[i], bmh); }, E, mt_s, wtot);
          int32_t* tab = po.mtile_start + h * (E + 1);
          for (int e = tid; e < E; e += 256) tab[e] = mt_s[e];
          if (tid == 0) tab[E] = mtot;
        }
        if (tid < kClaimSlots) po.mtile_start[2 * (E + 1) + tid] = 0;
      }
    }
  }
  const int tok0 = blockIdx.x * 4 * tpw;
  const int btok = block_tokens(T);
  const int blk = tok0 / btok;
  const int bt0 = blk * btok;
  const int c0 = MX ? 4 * (int)((long)(row16 / 4) * blockIdx.y / gridDim.y)
                    : (int)((long)row16 * blockIdx.y / gridDim.y);
  const int c1 = MX ? 4 * (int)((long)(row16 / 4) * (blockIdx.y + 1) / gridDim.y)
                    : (int)((long)row16 * (blockIdx.y + 1) / gridDim.y);
  const bool meta = blockIdx.y == 0;
  for (int e = tid; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  const int nblk = min(btok, T - bt0) * k;
  for (int a = tid; a < nblk; a += 256) {
    const int tl = a / k;
    atomicOr(&mask[topk_ids[(size_t)bt0 * k + a]], 1ull << tl);
  }
  __syncthreads();

  for (int i = 0; i < tpw; ++i) {
    const int t = tok0 + wave * tpw + i;
    if (t >= T) break;
    int row = 0;
    if (lane < k) {
      const int e = topk_ids[(size_t)t * k + lane];
      const int tl = t - bt0;
      const int rank = bases[(size_t)blk * E + e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
      row = (cap > 0 && rank >= cap) ? -1 : (po.counts ? off_s[e] : offsets[e]) + rank;
      if (meta) {
        token_row[(size_t)t * k + lane] = row;
        if (row >= 0) row_token[row] = t;
      }
    }
    if (!x_perm) continue;  // metadata only: the GEMM reads the token rows through row_token
    const u32x4* src = x + (size_t)t * row16;
    if constexpr (!MX) {
      for (int cb = c0; cb < c1; cb += kWave * kCopyUnroll) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int c = cb + u * kWave + lane;
          if (c < c1) v[u] = src[c];
        }
        for (int j = 0; j < k; ++j) {
          const int r = __shfl(row, j, kWave);
          if (r < 0) continue;  // dropped (uniform over the wave)
          u32x4* dst = x_perm + (size_t)r * row16;
          // the permuted rows are written once and read later by another kernel: a
          // nontemporal store streams them out (R1-shaped copy: 224 -> 180 us)
#pragma unroll
          for (int u = 0; u < kCopyUnroll; ++u) {
            const int c = cb + u * kWave + lane;
            if (c < c1) __builtin_nontemporal_store(v[u], dst + c);
          }
        }
      }
    } else {
      // wave-uniform trip count: the block-max shuffles need every lane of a group
      uint2* q = reinterpret_cast<uint2*>(x_perm);
      for (int cb = c0; cb < c1; cb += kWave * kCopyUnroll) {
        uint2 cv[kCopyUnroll];
        int sc[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int c = cb + u * kWave + lane;
          float f[8];
          unpack_bf16x8(__builtin_bit_cast(uint4, src[min(c, c1 - 1)]), f);
          cv[u] = mx_quantize8(f, &sc[u]);
        }
        for (int j = 0; j < k; ++j) {
          const int r = __shfl(row, j, kWave);
          if (r < 0) continue;  // dropped (uniform over the wave)
#pragma unroll
          for (int u = 0; u < kCopyUnroll; ++u) {
            const int c = cb + u * kWave + lane;
            if (c < c1) {
              q[(size_t)r * row16 + c] = cv[u];
              if ((c & 3) == 0) xs[(size_t)r * (row16 / 4) + (c >> 2)] = static_cast<uint8_t>(sc[u]);
            }
          }
        }
      }
    }
  }
}

hipError_t launch_permute(const void* x, int row16, const int32_t* ids, int T, int E, int k, int cap,
                          const int32_t* offsets, const int32_t* bases, void* x_perm, uint8_t* x_scale,
                          int32_t* row_token, int32_t* token_row, hipStream_t st,
                          const PermuteOffsets* po) {
  const PermuteOffsets pov = po ? *po : PermuteOffsets{nullptr, nullptr, 0, nullptr};
  if (pov.counts && E > 4 * 256) return hipErrorInvalidValue;
  // 4 tokens per wave for large T, 1 for small T (a workgroup's tokens always lie
  // in one ranking block); split columns until ~1024 workgroups
  const int tpw = T >= 4096 ? 4 : 1;
  const int gx = ceil_div(T, 4 * tpw);
  int cs = 1;
  while (x_perm && gx * cs < 1024 && row16 / (cs * 2) >= kWave) cs *= 2;
  if (x_scale) {  // MXFP8 dispatch of bf16 rows: row16 bf16 chunks -> row16 * 8 code bytes
    if (row16 % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_permute<true>, dim3(gx, cs), dim3(256), 0, st, static_cast<const u32x4*>(x), row16,
                       ids, T, E, k, tpw, cap, offsets, bases, static_cast<u32x4*>(x_perm), x_scale,
                       row_token, token_row, pov);
  } else {
    hipLaunchKernelGGL(k_permute<false>, dim3(gx, cs), dim3(256), 0, st, static_cast<const u32x4*>(x), row16,
                       ids, T, E, k, tpw, cap, offsets, bases, static_cast<u32x4*>(x_perm), nullptr,
                       row_token, token_row, pov);
  }
  return hipGetLastError();
}

}  // namespace moe
