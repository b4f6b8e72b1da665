// Permutation of token rows into expert-contiguous rows + routing metadata (step a4).
//
// The dispatcher permutes token activations into destination-contiguous
// buffers and attaches routing metadata; the receiver groups rows by expert
// (WideEP explainer (Kimi K3), "The router writes a network schedule").  On
// one GPU the destination is the expert itself, so one permutation does both.
// The buffer holds exactly T*k*D elements: the dispatch payload T x k x H x B
// of "Top-k multiplies traffic. Locality subtracts it." with every assignment
// local and no padding.
//
// Row order inside an expert's segment is ascending token id, independent of
// scheduling: row = base[block][e] + (number of lower tokens of the same
// 64-token block that picked e), the latter a popcount of a per-expert token
// bitmask built with order-independent LDS atomicOr.
#include "moe_kernels.h"

namespace moe {

constexpr int kPermTokPerWg = 16;  // 4 waves x 4 tokens
constexpr int kCopyUnroll = 4;

// x / x_perm are addressed in 16-byte units; a row is row16 units.
__global__ __launch_bounds__(256) void k_permute(const uint4* __restrict__ x, int row16,
                                                 const int32_t* __restrict__ topk_ids, int T,
                                                 int E, int k,
                                                 const int32_t* __restrict__ bases,
                                                 uint4* __restrict__ x_perm,
                                                 int32_t* __restrict__ row_token,
                                                 int32_t* __restrict__ token_row) {
  __shared__ unsigned long long mask[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok0 = blockIdx.x * kPermTokPerWg;
  const int blk = tok0 / kBlockTok;
  const int bt0 = blk * kBlockTok;
  for (int e = tid; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  const int nblk = min(kBlockTok, T - bt0) * k;
  for (int a = tid; a < nblk; a += 256) {
    const int tl = a / k;
    atomicOr(&mask[topk_ids[(size_t)bt0 * k + a]], 1ull << tl);
  }
  __syncthreads();

  for (int i = 0; i < kPermTokPerWg / 4; ++i) {
    const int t = tok0 + wave * (kPermTokPerWg / 4) + i;
    if (t >= T) break;
    int row = 0;
    if (lane < k) {
      const int e = topk_ids[(size_t)t * k + lane];
      const int tl = t - bt0;
      const int rank = __popcll(mask[e] & ((1ull << tl) - 1ull));
      row = bases[(size_t)blk * E + e] + rank;
      token_row[(size_t)t * k + lane] = row;
      row_token[row] = t;
    }
    const uint4* src = x + (size_t)t * row16;
    for (int c0 = 0; c0 < row16; c0 += kWave * kCopyUnroll) {
      uint4 v[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < row16) v[u] = src[c];
      }
      for (int j = 0; j < k; ++j) {
        const int r = __shfl(row, j, kWave);
        uint4* dst = x_perm + (size_t)r * row16;
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int c = c0 + u * kWave + lane;
          if (c < row16) dst[c] = v[u];
        }
      }
    }
  }
}

hipError_t launch_permute(const void* x, int row16, const int32_t* ids, int T, int E, int k,
                          const int32_t* bases, void* x_perm, int32_t* row_token,
                          int32_t* token_row, hipStream_t st) {
  hipLaunchKernelGGL(k_permute, dim3(ceil_div(T, kPermTokPerWg)), dim3(256), 0, st,
                     static_cast<const uint4*>(x), row16, ids, T, E, k, bases,
                     static_cast<uint4*>(x_perm), row_token, token_row);
  return hipGetLastError();
}

}  // namespace moe
