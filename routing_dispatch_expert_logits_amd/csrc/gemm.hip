// Grouped expert GEMMs (step a5) and the dense projections built on them
// (gate scores, step a1; latent down/up projections, step a7).
//
// Expert e owns rows [offsets[e], offsets[e+1]) of the permuted buffer; one
// launch covers every expert with its own row count, and an expert with no
// rows contributes no tile ("Three Parameter Counts...", table of "Which
// optimizations need a task-level gate").  The tile table is on the device:
// mtile_start[e] = sum_{e' < e} ceil(rows_e' / BM), so a workgroup finds its
// (expert, m-tile, n-tile) with a binary search and the grid is sized from
// host-known bounds only.
//
// Tile order: expert-major, then n-tile (or a group of n-tiles), then m-tile, so
// the tiles that share an expert's weights and rows run together; logical tiles are dealt to the 8 XCDs
// in contiguous chunks (workgroup i runs on XCD i % 8), keeping each expert's
// working set in one XCD's L2.
//
// bf16 path: v_mfma_f32_16x16x32_bf16, fp32 accumulate.  Lane l of a 16x16x32
// MFMA supplies A[l % 16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l % 16] and
// receives D[4*(l/16) .. +4][l % 16].  Because every weight is stored
// output-major (K contiguous), both operands are 16-byte K-runs.
#include "moe_kernels.h"

namespace moe {

// ------------------------------------------------------------------ tile decode

struct TileCoord {
  int e, row0, rows, n0;
};

// Logical tile L of a grouped GEMM (L < mtile_start[E] * ceil(N / BN)).
template <int BM, int BN, int G>
__device__ __forceinline__ TileCoord grouped_tile(const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ mtile_start, int E, int N,
                                                  int L) {
  const int NT = ceil_div(N, BN);
  const int e = upper_index(mtile_start, E, L / NT);
  const int mt0 = mtile_start[e];
  const int mte = mtile_start[e + 1] - mt0;
  const int local = L - mt0 * NT;
  int n_idx, m_idx;
  if constexpr (G == 1) {
    n_idx = local / mte;
    m_idx = local - n_idx * mte;
  } else {
    const int grp = local / (G * mte), r = local - grp * (G * mte);
    const int ng = min(G, NT - grp * G);  // n-tiles in this group
    m_idx = r / ng;
    n_idx = grp * G + (r - m_idx * ng);
  }
  TileCoord tc;
  tc.e = e;
  tc.row0 = offsets[e] + m_idx * BM;
  tc.rows = min(BM, offsets[e + 1] - tc.row0);
  tc.n0 = n_idx * BN;
  return tc;
}

// Returns false when this workgroup has no tile.  Within an expert, tiles run in
// groups of G consecutive n-tiles; inside a group the m-tile index is outer, so
// the G tiles reading one m-tile's rows are adjacent and each weight panel is
// reused G tiles later.
template <int BM, int BN, int G = 1>
__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ offsets,
                                            const int32_t* __restrict__ mtile_start, int E, int M,
                                            int N, TileCoord& tc) {
  const int NT = ceil_div(N, BN);
  const int total_mt = offsets ? mtile_start[E] : ceil_div(M, BM);
  const int total = total_mt * NT;
  const int per_xcd = ceil_div(total, 8);
  const int slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  if (slot >= per_xcd) return false;
  const int L = xcd * per_xcd + slot;
  if (L >= total) return false;
  if (offsets) {
    tc = grouped_tile<BM, BN, G>(offsets, mtile_start, E, N, L);
  } else {
    const int n_idx = L / total_mt, m_idx = L - n_idx * total_mt;
    tc.e = 0;
    tc.row0 = m_idx * BM;
    tc.rows = min(BM, M - tc.row0);
    tc.n0 = n_idx * BN;
  }
  return true;
}

// SiLU(g) * u = g * u / (1 + e^-g), with e^-g = 2^(-g log2 e) from the hardware exp2 and
// the hardware reciprocal (each within about one fp32 ulp, far below the bf16 rounding
// of the intermediate).  A very negative g overflows e^-g to inf and its reciprocal to
// 0, so the product is 0, as SiLU tends to.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.f + e) * u;
}

template <int EPI>
__device__ __forceinline__ void epi_store(void* C, size_t idx, float v0, float v1, const float* bias,
                                          int col) {
  if constexpr (EPI == EPI_BF16) {
    static_cast<uint16_t*>(C)[idx] = f32_to_bf16(v0);
  } else if constexpr (EPI == EPI_SWIGLU_BF16) {
    static_cast<uint16_t*>(C)[idx] = f32_to_bf16(silu_mul(v0, v1));
  } else if constexpr (EPI == EPI_F32) {
    static_cast<float*>(C)[idx] = v0;
  } else if constexpr (EPI == EPI_SWIGLU_F32) {
    static_cast<float*>(C)[idx] = silu_mul(v0, v1);
  } else {  // EPI_F32_BIAS
    static_cast<float*>(C)[idx] = bias ? v0 + bias[col] : v0;
  }
}

// ------------------------------------------------------------------ bf16 prefill kernel
// Workgroup tile BM x BN (x NB weight matrices sharing the A tile), 4 waves in
// 2 x 2, K-step 64 staged through LDS (rows padded to 80 elements: 160-byte rows
// let one MFMA operand read of 16 rows run at full LDS rate on gfx950), next
// step's global loads in flight during the current step's MFMAs.

constexpr int kPBK = 64;

// MINW: waves per SIMD the register budget must allow (2 -> two workgroups per CU);
// PAD: LDS row padding in bf16 elements.
template <int BM, int BN, int NB, int EPI, int MINW = 1, int PAD = 16>
__global__ __launch_bounds__(256, MINW) void k_gemm_prefill(
    const uint16_t* __restrict__ A, int M, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ mtile_start, int E, int N, int K) {
  constexpr int kPLD = kPBK + PAD;
  constexpr int TM = BM / 2, TN = BN / 2;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_PER = BM * 8 / 256, B_PER = BN * 8 / 256;
  static_assert(A_PER >= 1 && B_PER >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kPLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[NB][BN * kPLD];

  TileCoord tc;
  if (!decode_tile<BM, BN>(offsets, mtile_start, E, M, N, tc)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const uint16_t* B0e = B0 + (size_t)tc.e * N * K;
  const uint16_t* B1e = NB > 1 ? B1 + (size_t)tc.e * N * K : B0e;

  // loader mapping: chunk i of this thread is row (tid / 8) + 32 i, K-offset 8 * (tid % 8);
  // source rows are clamped into the tile so no load leaves its expert's segment
  const int lrow = tid >> 3, lk = (tid & 7) * 8;
  uint32_t aoff[A_PER], boff[B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i)
    aoff[i] = (uint32_t)(tc.row0 + min(lrow + 32 * i, tc.rows - 1));
#pragma unroll
  for (int i = 0; i < B_PER; ++i) boff[i] = (uint32_t)min(tc.n0 + lrow + 32 * i, N - 1);
  const int lds0 = lrow * kPLD + lk;
  auto a_src = [&](int i, int k0) {
    return reinterpret_cast<const u32x4*>(A + (size_t)aoff[i] * K + lk + k0);
  };
  auto b_src = [&](int nb, int i, int k0) {
    return reinterpret_cast<const u32x4*>((nb == 0 ? B0e : B1e) + (size_t)boff[i] * K + lk + k0);
  };

  f32x4 acc[NB][FM][FN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[nb][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[A_PER], rb[NB][B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) ra[i] = *a_src(i, 0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < B_PER; ++i) rb[nb][i] = *b_src(nb, i, 0);

  const int arow = wm * TM + (lane & 15);
  const int brow = wn * TN + (lane & 15);
  const int kofs = (lane >> 4) * 8;

  for (int k0 = 0; k0 < K; k0 += kPBK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_PER; ++i) *reinterpret_cast<u32x4*>(&sA[lds0 + 32 * i * kPLD]) = ra[i];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < B_PER; ++i) *reinterpret_cast<u32x4*>(&sB[nb][lds0 + 32 * i * kPLD]) = rb[nb][i];
    __syncthreads();
    {  // next step's loads (the last step re-reads its own slice, keeping the loop branch-free)
      const int kn = min(k0 + kPBK, K - kPBK);
#pragma unroll
      for (int i = 0; i < A_PER; ++i) ra[i] = *a_src(i, kn);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < B_PER; ++i) rb[nb][i] = *b_src(nb, i, kn);
    }
#pragma unroll
    for (int ks = 0; ks < kPBK; ks += 32) {
      bf16x8 af[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sA[(arow + fm * 16) * kPLD + ks + kofs]));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const bf16x8 bf =
              as_bf16x8(*reinterpret_cast<const u32x4*>(&sB[nb][(brow + fn * 16) * kPLD + ks + kofs]));
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
            acc[nb][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bf, acc[nb][fm][fn], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each 16x16 fragment
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * TM + fm * 16 + (lane >> 4) * 4 + i;
        const int c = tc.n0 + wn * TN + fn * 16 + (lane & 15);
        if (r < tc.rows && c < N)
          epi_store<EPI>(C, (size_t)(tc.row0 + r) * N + c, acc[0][fm][fn][i],
                         NB > 1 ? acc[NB - 1][fm][fn][i] : 0.f, nullptr, c);
      }
}

// ------------------------------------------------------------------ bf16 pipelined kernel
// Wave-specialised variant of the tile kernel: MW MFMA waves (64 x TN tiles, two
// per SIMD when MW = 8) and 2 loader waves per workgroup.  The loader waves copy
// each K-step's A and B tiles straight from global memory into an S-stage LDS
// ring with global_load_lds_dwordx4 (no register staging) and run up to S-1
// stages ahead; the MFMA waves only read LDS.  One barrier per K-step hands a
// stage to the MFMA waves and the freed stage back to the loaders.  Because only
// the loader waves issue the LDS DMA, the MFMA waves' LDS reads never wait for
// loads of later stages.
//
// LDS layout: a tile is rows of BK bf16 in 16-byte chunks; chunk c of row r sits
// at chunk slot c ^ swz(r).  Measured on gfx950 (ds_read_b128 of the 16 rows one
// MFMA operand touches, at one chunk index): 128-byte rows (BK = 64) run at full
// LDS rate (~200 B/clk/CU) with swz(r) = r & 7, 64-byte rows (BK = 32) with
// swz(r) = (r >> 1) & 3; unswizzled rows run at a half or a quarter of that.  A
// DMA instruction fills 1 KB: 64 / (BK / 8) consecutive rows (lane i -> row
// i / (BK / 8), slot i % (BK / 8)).

template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 64) return r & 7;
  else return (r >> 1) & 3;
}

// The LDS-DMA builtin takes a global-address-space source and an LDS
// destination; spelling both casts out keeps the host compilation pass of the
// kernel valid (it otherwise drops the kernel's host stub).
typedef const __attribute__((address_space(1))) void* gas_ptr;
typedef __attribute__((address_space(3))) void* las_ptr;

// s_waitcnt immediate that waits until at most n vector-memory ops are outstanding
// (vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at "no wait").
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
static_assert(waitcnt_vm(24) == 0x4F78 && waitcnt_vm(0) == 0x0F70, "s_waitcnt encoding");

//
// F8 = true: MXFP8 operands (E4M3 codes, one E8M0 scale per 32 elements along K,
// mx.a / mx.b0 / mx.b1 the [rows x K/32] scale arrays).  The code matrices are
// passed as 16-bit pairs with K = D / 2, so a K-step is still 128 bytes per row
// and the loaders and LDS layout are those of the bf16 kernel.  The loader waves
// also copy each stage's scales (4 bytes per row: the step's four blocks) into a
// region after the B tiles with 4-byte LDS DMA.  The MFMA waves feed one
// v_mfma_scale_f32_16x16x128_f8f6f4 per fragment and K-step: lane l (g = l / 16)
// supplies the 16-byte chunks g and 4 + g of its row's K-step (K elements
// 16g..16g+15 and 64+16g..64+16g+15) and the E8M0 scale of block g of that step.
template <int BM, int BN, int NB, int EPI, int S, int MW = 4, int BK = 64, int G = 1, bool F8 = false>
__global__ __launch_bounds__(MW * 64 + 128) void k_gemm_ws(
    const uint16_t* __restrict__ A, int M, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ mtile_start, int E, int N, int K, MxScales mx) {
  static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile 128/256 x 128/256");
  static_assert(BK == 32 || BK == 64, "K-step 32 or 64");
  static_assert(!F8 || BK == 64, "MXFP8 K-steps are 128 codes");
  constexpr int WM = BM / 64;                     // MFMA waves along M (64 rows each)
  constexpr int WN = MW / WM;                     // MFMA waves along N
  static_assert(WM * WN == MW && WN >= 1, "wave grid");
  constexpr int TM = 64, TN = BN / WN, FM = 4, FN = TN / 16;
  constexpr int CH = BK / 8;                      // 16-byte chunks per LDS row
  constexpr int RPQ = 64 / CH;                    // rows per DMA instruction
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  constexpr int SC_BYTES = F8 ? (BM + NB * BN) * 4 : 0;        // MXFP8 scales per stage
  constexpr int STAGE = A_ELEMS + NB * B_ELEMS + SC_BYTES / 2;  // 16-bit elements per stage
  constexpr int QA = BM / RPQ, QB = BN / RPQ;     // DMA instructions per A / B tile
  constexpr int NQ = QA + NB * QB;                // DMA instructions per stage
  constexpr int NQP = NQ / 2;                     // per loader wave
  constexpr int SQA = F8 ? BM / 64 : 0, SQB = F8 ? BN / 64 : 0;  // 4-byte scale DMAs (64 rows each)
  constexpr int NSP = (SQA + NB * SQB) / 2;       // scale DMAs per loader wave
  static_assert((SQA + NB * SQB) % 2 == 0, "scale DMAs split over two loader waves");
  constexpr int NQW = NQP + NSP;                  // vector-memory ops per stage per loader wave
  static_assert(S >= 2 && S <= 6 && (S - 2) * NQW <= 63, "outstanding loads fit vmcnt");
  __shared__ __attribute__((aligned(16))) uint16_t lds[S * STAGE];

  TileCoord tc;
  if (!decode_tile<BM, BN, G>(offsets, mtile_start, E, M, N, tc)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nsteps = K / BK;

  if (wave >= MW) {
    // ---------------- loader waves
    const int p = wave - MW;
    const uint16_t* src[NQP];
    int ldsoff[NQP];
#pragma unroll
    for (int j = 0; j < NQP; ++j) {
      const int q = p * NQP + j;       // instruction index within the stage
      if (q < QA) {                    // A tile rows RPQ*q ..
        const int r = q * RPQ + lane / CH;
        const int c = (lane % CH) ^ swz<BK>(r);
        src[j] = A + (size_t)(tc.row0 + min(r, tc.rows - 1)) * K + c * 8;
        ldsoff[j] = q * 512;
      } else {                         // B tile nb, rows RPQ*qq ..
        const int nb = (q - QA) / QB, qq = (q - QA) % QB;
        const int r = qq * RPQ + lane / CH;
        const int c = (lane % CH) ^ swz<BK>(r);
        const uint16_t* Bm = nb == 0 ? B0 : B1;
        src[j] = Bm + ((size_t)tc.e * N + min(tc.n0 + r, N - 1)) * K + c * 8;
        ldsoff[j] = A_ELEMS + nb * B_ELEMS + qq * 512;
      }
    }
    // MXFP8 scales: lane i of DMA j copies the step's 4 scale bytes of row i of its
    // 64-row group (scale rows are K / 16 bytes: K counts 16-bit pairs)
    const uint8_t* ssrc[NSP > 0 ? NSP : 1];
    int sldsoff[NSP > 0 ? NSP : 1];
    if constexpr (F8) {
      const int srow = K / 16;
#pragma unroll
      for (int j = 0; j < NSP; ++j) {
        const int q = p * NSP + j;
        if (q < SQA) {
          const int r = q * 64 + lane;
          ssrc[j] = mx.a + (size_t)(tc.row0 + min(r, tc.rows - 1)) * srow;
          sldsoff[j] = (A_ELEMS + NB * B_ELEMS) * 2 + q * 256;
        } else {
          const int nb = (q - SQA) / SQB, qq = (q - SQA) % SQB;
          const int r = qq * 64 + lane;
          ssrc[j] = (nb == 0 ? mx.b0 : mx.b1) + ((size_t)tc.e * N + min(tc.n0 + r, N - 1)) * srow;
          sldsoff[j] = (A_ELEMS + NB * B_ELEMS) * 2 + BM * 4 + nb * BN * 4 + qq * 256;
        }
      }
    }
    auto issue = [&](int st) {
      const int base = (st % S) * STAGE;
#pragma unroll
      for (int j = 0; j < NQP; ++j)
        __builtin_amdgcn_global_load_lds((gas_ptr)(src[j] + st * BK), (las_ptr)&lds[base + ldsoff[j]],
                                         16, 0, 0);
      if constexpr (F8) {
#pragma unroll
        for (int j = 0; j < NSP; ++j)
          __builtin_amdgcn_global_load_lds((gas_ptr)(ssrc[j] + st * 4),
                                           (las_ptr)(reinterpret_cast<uint8_t*>(lds) + base * 2 + sldsoff[j]),
                                           4, 0, 0);
      }
    };
    // Up to S-1 stages in flight.  wait_behind(n): the oldest outstanding stage has
    // landed once at most n later stages (n * NQW loads) are still in flight.
    auto wait_behind = [](int n) {
      if (n >= 4) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * NQW < 63 ? 4 * NQW : 63));
      else if (n == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * NQW < 63 ? 3 * NQW : 63));
      else if (n == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NQW < 63 ? 2 * NQW : 63));
      else if (n == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NQW));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    };
    const int pre = min(S - 1, nsteps);               // stages issued before the loop
    for (int st = 0; st < pre; ++st) issue(st);
    wait_behind(pre - 1);                             // stage 0 landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int s = 0; s < nsteps; ++s) {
      if (s + S - 1 < nsteps) issue(s + S - 1);       // into the stage freed by step s - 1
      // stage s+1 must land; later issued stages are s+2 .. min(s+S-1, nsteps-1)
      wait_behind(max(0, min(s + S - 1, nsteps - 1) - (s + 1)));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    return;
  }

  // ---------------- MFMA waves
  const int wm = wave / WN, wn = wave % WN;
  // a wave whose 64 rows all lie past the tile's valid rows only keeps the barrier
  // cadence (one barrier before the loop, one per K-step)
  if (wm * TM >= tc.rows) {
    for (int s = 0; s <= nsteps; ++s) __syncthreads();
    return;
  }
  f32x4 acc[NB][FM][FN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[nb][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
  // element offsets of this lane's operand chunks inside a stage, per 32-wide substep
  constexpr int NH = BK / 32;
  int aoffs[NH][FM], boffs[NH][FN];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int c = h * 4 + (lane >> 4);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int r = wm * TM + fm * 16 + (lane & 15);
      aoffs[h][fm] = r * BK + ((c ^ swz<BK>(r)) << 3);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int r = wn * TN + fn * 16 + (lane & 15);
      boffs[h][fn] = A_ELEMS + r * BK + ((c ^ swz<BK>(r)) << 3);
    }
  }
  // Operands are double-buffered in registers: the LDS reads of the next 32-wide
  // substep are issued between the MFMAs of the current one, and the first reads of
  // stage s+1 go out right after the barrier that releases it, ahead of stage s's
  // last MFMAs.  So LDS reads overlap the MFMA pipe instead of preceding it.
  struct Ops {
    bf16x8 a[FM];
    bf16x8 b[NB][FN];
  };
  constexpr int NR = FM + NB * FN, NM = NB * FN * FM;   // reads and MFMAs per substep
  auto rd = [&](Ops& o, const uint16_t* base, int h) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) o.a[fm] = as_bf16x8(*reinterpret_cast<const u32x4*>(base + aoffs[h][fm]));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        o.b[nb][fn] = as_bf16x8(*reinterpret_cast<const u32x4*>(base + nb * B_ELEMS + boffs[h][fn]));
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[nb][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[fm], o.b[nb][fn], acc[nb][fm][fn], 0, 0, 0);
  };
  // one MFMA, one LDS read, alternating while reads remain, then the other MFMAs
  auto interleave = [] {
#pragma unroll
    for (int i = 0; i < (NR < NM ? NR : NM); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
  };
  static_assert(NH == 1 || NH == 2, "one or two substeps per K-step");
  // Double-buffering needs a second operand set in registers; tiles whose
  // accumulators leave no room for it (VGPRs per wave: 512 / waves per SIMD) read
  // each substep's operands just before its MFMAs instead.
  constexpr int kWavesPerSimd = (MW + 2 + 3) / 4;
  constexpr int kVgprBudget = (512 / kWavesPerSimd) & ~7;
  constexpr bool kDoubleBuffer = NM * 4 + 2 * NR * 4 + 40 <= kVgprBudget;
  if constexpr (F8) {
    // per K-step: both chunks of every fragment, the fragments' block scales, one
    // scaled MFMA per fragment pair
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    constexpr int SCB = (A_ELEMS + NB * B_ELEMS) * 2;  // scale region, bytes into the stage
    const int g = lane >> 4;
    int sa_off[FM], sb_off[NB][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sa_off[fm] = SCB + (wm * TM + fm * 16 + (lane & 15)) * 4 + g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        sb_off[nb][fn] = SCB + BM * 4 + nb * BN * 4 + (wn * TN + fn * 16 + (lane & 15)) * 4 + g;
    __syncthreads();  // stage 0 has landed
    for (int s = 0; s < nsteps; ++s) {
      const uint16_t* base = lds + (s % S) * STAGE;
      const uint8_t* base8 = reinterpret_cast<const uint8_t*>(base);
      // B fragments and all scales first, then A fragment by fragment, and the MFMAs
      // fragment-row by fragment-row, so each row's MFMAs wait only for their own A
      u32x4 a0[FM], a1[FM], b0[NB][FN], b1[NB][FN];
      int sa[FM], sb[NB][FN];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          b0[nb][fn] = *reinterpret_cast<const u32x4*>(base + nb * B_ELEMS + boffs[0][fn]);
          b1[nb][fn] = *reinterpret_cast<const u32x4*>(base + nb * B_ELEMS + boffs[1][fn]);
          sb[nb][fn] = base8[sb_off[nb][fn]];
        }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) sa[fm] = base8[sa_off[fm]];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        a0[fm] = *reinterpret_cast<const u32x4*>(base + aoffs[0][fm]);
        a1[fm] = *reinterpret_cast<const u32x4*>(base + aoffs[1][fm]);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0[fm], a1[fm], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const i32x8 bv = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0[nb][fn], b1[nb][fn], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[nb][fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[nb][fm][fn], 0, 0, 0,
                                                                               sa[fm], 0, sb[nb][fn]);
          }
      }
      __syncthreads();  // every MFMA wave has read stage s; stage s+1 has landed
    }
  } else if constexpr (!kDoubleBuffer) {
    __syncthreads();  // stage 0 has landed
    for (int s = 0; s < nsteps; ++s) {
      const uint16_t* base = lds + (s % S) * STAGE;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        Ops o;
        rd(o, base, h);
        mma(o);
      }
      __syncthreads();  // every MFMA wave has read stage s; stage s+1 has landed
    }
  } else {
    Ops o0, o1;
    __syncthreads();  // stage 0 has landed
    rd(o0, lds, 0);
    for (int s = 0; s < nsteps; ++s) {
      // the reads after the barrier fetch stage s+1; on the last step they read a
      // stale (in-bounds) stage that no MFMA consumes
      const uint16_t* nxt = lds + ((s + 1) % S) * STAGE;
      if constexpr (NH == 2) {
        rd(o1, lds + (s % S) * STAGE, 1);
        mma(o0);
        interleave();
        __syncthreads();  // every MFMA wave has read stage s; stage s+1 has landed
        rd(o0, nxt, 0);
        mma(o1);
        interleave();
      } else {
        __syncthreads();
        rd(o1, nxt, 0);
        mma(o0);
        interleave();
        o0 = o1;
      }
    }
  }

#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * TM + fm * 16 + (lane >> 4) * 4 + i;
        const int c = tc.n0 + wn * TN + fn * 16 + (lane & 15);
        if (r < tc.rows && c < N)
          epi_store<EPI>(C, (size_t)(tc.row0 + r) * N + c, acc[0][fm][fn][i],
                         NB > 1 ? acc[NB - 1][fm][fn][i] : 0.f, nullptr, c);
      }
}

// ------------------------------------------------------------------ persistent variant
// k_gemm_wsp: the wave-specialised kernel as a persistent kernel for the expert
// GEMMs.  One workgroup per CU; workgroup i runs on XCD i % 8 and takes the tiles
// of that XCD's contiguous chunk of logical tiles one at a time, in order, from the
// chunk's claim counter (claim[i % 8], an agent-scope atomic).  So the 32 CUs of an
// XCD work through its chunk in the order the hardware would have dispatched
// one-tile workgroups (the tiles sharing an expert's weights run together), a CU
// that runs slow simply takes fewer tiles, and there is no per-tile dispatch, launch
// or pipeline fill: the loader waves run ahead across tile boundaries, so the next
// tile's first stages are in flight while the MFMA waves store the previous one.  An
// eleventh wave makes the claims (and, for gathered rows, DMAs the next tile's token
// row indices into LDS), so the loader waves never wait on anything but their own
// LDS DMA: a claim's result in a loader wave would make the compiler drain its DMA.
// Each workgroup decodes the tile coordinates once into an LDS table (every tile
// when they fit, else its own XCD's chunk).  A workgroup whose chunk is done takes
// tiles left in other XCDs' chunks, from the chunk with the most left (the XCDs
// finish a few percent apart); a taken tile outside its table is decoded from the
// m-tile table in memory, and the scheduler wave publishes every claimed tile's
// coordinates in LDS.  Tiles, K-steps, LDS layout and MFMA order are those of
// k_gemm_ws, so the results are the same bits.  The claim counters must be zero at launch: the m-tile table kernels
// (k_offsets, k_route_small, k_single_group) clear them.

// Chunk entries an LDS table can hold (4 bytes each: expert | m-tile << 10 | n-tile << 22).
template <bool F8>
constexpr int wsp_table_cap() { return F8 ? 2624 : 3520; }
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0) (vmcnt, expcnt not waited)

// Whether the persistent kernel takes a GEMM of at most `tiles` tiles of BM rows, over
// at most M rows per expert, N columns and K 16-bit columns: the XCD chunk fits the LDS
// table, every tile coordinate fits its field of a table entry (expert 10 bits, m-tile
// 12 bits, n-tile 10 bits), and a tile has at least 4 K-steps (the scheduler wave
// publishes the next tile's claim by K-step nsteps - 4, the loader waves read it at
// K-step nsteps - 2).
template <bool F8>
static inline bool wsp_fits(long tiles, int M, int BM, int E, int N, int K) {
  return (tiles + 7) / 8 <= wsp_table_cap<F8>() && E <= 1024 && ceil_div(M, BM) <= 4096 &&
         ceil_div(N, 128) <= 1024 && K % 64 == 0 && K / 64 >= 4;
}

template <int BM, int BN, int NB, int EPI, int S, int MW = 8, bool F8 = false>
__global__ __launch_bounds__(MW * 64 + 192) void k_gemm_wsp(
    const uint16_t* __restrict__ A, int M, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ mtile_start, int E, int N, int K, MxScales mx, int32_t* __restrict__ claim,
    const int32_t* __restrict__ gather) {
  constexpr int BK = 64;
  constexpr int WM = BM / 64, WN = MW / WM;
  static_assert(WM * WN == MW && WN >= 1, "wave grid");
  constexpr int TM = 64, TN = BN / WN, FM = 4, FN = TN / 16;
  constexpr int CH = BK / 8, RPQ = 64 / CH;
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  constexpr int SC_BYTES = F8 ? (BM + NB * BN) * 4 : 0;
  constexpr int STAGE = A_ELEMS + NB * B_ELEMS + SC_BYTES / 2;
  constexpr int QA = BM / RPQ, QB = BN / RPQ, NQ = QA + NB * QB, NQP = NQ / 2;
  constexpr int SQA = F8 ? BM / 64 : 0, SQB = F8 ? BN / 64 : 0;
  constexpr int NSP = (SQA + NB * SQB) / 2;
  static_assert((SQA + NB * SQB) % 2 == 0, "scale DMAs split over two loader waves");
  constexpr int NQW = NQP + NSP;  // vector-memory ops per stage per loader wave
  static_assert(S == 3 && NQW <= 63, "three stages: one stage in flight behind the one landing");
  constexpr int CAP = wsp_table_cap<F8>();
  constexpr int NTHR = MW * 64 + 192;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S * STAGE];
  __shared__ uint32_t table[CAP];
  __shared__ int claimed[4];       // logical index of tile ti of this workgroup at [ti % 4], -1 past the end
  __shared__ uint32_t centry[4];   // its packed coordinates (expert | m-tile << 10 | n-tile << 22)
  __shared__ int32_t grow[2][BM];  // gathered rows: token row of each tile row, tile ti at [ti % 2]

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = ceil_div(N, BN);
  const int total = mtile_start[E] * NT;
  const int per_xcd = ceil_div(total, 8);
  const int xcd = blockIdx.x & 7;
  const int lo = xcd * per_xcd, chunk = max(0, min(per_xcd, total - lo));  // chunk <= CAP by wsp_fits
  if (total == 0) return;
  // The table holds every tile when they fit, else this XCD's chunk only.
  const bool all = total <= CAP;
  const int tlo = all ? 0 : lo, tcount = all ? total : chunk;
  // table[L - tlo] for logical tile L in logical order (expert-major, then n-tile, then m-tile)
  for (int e = tid; e < E; e += NTHR) {
    const int mt0 = mtile_start[e], mte = mtile_start[e + 1] - mt0;
    const int b = max(0, tlo - mt0 * NT), f = min(mte * NT, tlo + tcount - mt0 * NT);
    for (int local = b; local < f; ++local) {
      const int n = local / mte, m = local - n * mte;
      table[mt0 * NT + local - tlo] = (uint32_t)e | ((uint32_t)m << 10) | ((uint32_t)n << 22);
    }
  }
  __syncthreads();
  const int nsteps = K / BK;

  // packed coordinates V of a tile: expert, first row, rows, first column (wave-uniform)
#define MOE_WSP_COORDS(V, e, r0, rows, n0)                                                     \
  {                                                                                            \
    const uint32_t v_ = (V);                                                                   \
    e = __builtin_amdgcn_readfirstlane((int)(v_ & 1023u));                                     \
    const int m_ = __builtin_amdgcn_readfirstlane((int)((v_ >> 10) & 4095u));                  \
    n0 = __builtin_amdgcn_readfirstlane((int)(v_ >> 22)) * BN;                                 \
    r0 = offsets[e] + m_ * BM;                                                                 \
    rows = min(BM, offsets[e + 1] - r0);                                                       \
  }

  if (wave == MW + 2) {
    // ---------------- scheduler wave: tile claims, and the token rows of gathered tiles.
    // Its vmcnt waits for the claim's result are its own: the loader waves never wait
    // on anything but their LDS DMA.
    // The logical tile for a claim `own` made on this XCD's counter, or -1 when no tile
    // is left.  Each failed steal meets a counter already past its chunk, which every
    // later agent-scope load of it shows, so the loop ends after at most 9 rounds.
    auto take = [&](int own) -> int {
      if (own < chunk) return lo + own;
      for (int round = 0; round < 16; ++round) {
        int left = -1;
        if (lane < 8) {
          const int c = __hip_atomic_load(&claim[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          left = max(0, min(per_xcd, total - lane * per_xcd)) - c;
        }
        int best = left, who = lane;
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          const int l2 = __shfl_xor(best, o), w2 = __shfl_xor(who, o);
          if (l2 > best || (l2 == best && w2 < who)) {
            best = l2;
            who = w2;
          }
        }
        best = __builtin_amdgcn_readfirstlane(best);
        who = __builtin_amdgcn_readfirstlane(who);
        if (best <= 0) return -1;
        int t = 0;
        if (lane == 0) t = atomicAdd(&claim[who], 1);
        t = __builtin_amdgcn_readfirstlane(t);
        if (t < max(0, min(per_xcd, total - who * per_xcd))) return who * per_xcd + t;
      }
      return -1;
    };
    // The packed coordinates of logical tile L: from the LDS table when it holds L, else
    // (a tile taken from another XCD's chunk) from the m-tile table in memory: the expert
    // is the last e with mtile_start[e] <= L / NT (the table is non-decreasing, so those
    // e form a prefix, counted 64 at a time with a ballot), then the table's own decode.
    auto entry_of = [&](int L) -> uint32_t {
      if (L >= tlo && L < tlo + tcount) return table[L - tlo];
      const int mrow = L / NT;
      int p = 0;
      for (int base = 0; base <= E; base += 64) {
        const int idx = base + lane;
        const int c = __popcll(__ballot(idx <= E && mtile_start[min(idx, E)] <= mrow));
        p += c;
        if (c < 64) break;
      }
      const int e = p - 1;
      const int mt0 = mtile_start[e], mte = mtile_start[e + 1] - mt0;
      const int local = L - mt0 * NT, n = local / mte, m = local - n * mte;
      return (uint32_t)e | ((uint32_t)m << 10) | ((uint32_t)n << 22);
    };
    // publish tile ti's claim and coordinates, and (gathered rows) DMA its token-row
    // indices into grow
    auto publish = [&](int ti, int L) {
      const uint32_t ent = L >= 0 ? entry_of(L) : 0u;
      if (lane == 0) {
        claimed[ti & 3] = L;
        centry[ti & 3] = ent;
      }
      if (gather && L >= 0) {
        int g_e, g_r0, g_rows, g_n0;
        MOE_WSP_COORDS(ent, g_e, g_r0, g_rows, g_n0)
        (void)g_e;
        (void)g_n0;
#pragma unroll
        for (int h = 0; h < BM / 64; ++h)
          __builtin_amdgcn_global_load_lds((gas_ptr)(gather + g_r0 + min(h * 64 + lane, g_rows - 1)),
                                           (las_ptr)&grow[ti & 1][h * 64], 4, 0, 0);
      }
    };
    {
      int t = 0;
      if (lane == 0) t = atomicAdd(&claim[xcd], 1);
      publish(0, take(__builtin_amdgcn_readfirstlane(t)));
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();  // the first tile's claim and token rows are in LDS
    if (claimed[0] < 0) return;
    // The next tile's claim goes out at K-step 0 of a tile and is published at K-step P
    // (its DMA done by P + 1); the loader waves read it when they start the next tile's
    // stages, at K-step nsteps - 2 (nsteps >= 4), the MFMA waves at the tile's start.
    const int P = min(2, nsteps - 4);
    __builtin_amdgcn_s_barrier();  // stage 0 has landed (the loaders' barrier)
    asm volatile("" ::: "memory");
    int pend = 0;
    for (int ti = 0;; ++ti) {
      if (claimed[ti & 3] < 0) break;
      for (int st = 0; st < nsteps; ++st) {
        if (st == 0 && lane == 0) pend = atomicAdd(&claim[xcd], 1);
        if (st == P) publish(ti + 1, take(__builtin_amdgcn_readfirstlane(pend)));
        if (st == P + 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the row-index DMA landed
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // claimed[] written
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
    return;
  }
  __syncthreads();  // the first tile's claim (and token rows) are in LDS
  if (claimed[0] < 0) return;  // the same value for every wave

  if (wave >= MW) {
    // ---------------- loader waves: stage f of the flattened (tile, K-step) sequence
    const int p = wave - MW;
    const uint16_t* src[NQP];
    int ldsoff[NQP];
    const uint8_t* ssrc[NSP > 0 ? NSP : 1];
    int sldsoff[NSP > 0 ? NSP : 1];
#define MOE_WSP_SET_TILE(ti)                                                                          \
  {                                                                                                   \
    int t_e, t_r0, t_rows, t_n0;                                                                      \
    MOE_WSP_COORDS(centry[(ti) & 3], t_e, t_r0, t_rows, t_n0)                                         \
    _Pragma("unroll") for (int j = 0; j < NQP; ++j) {                                                 \
      const int q = p * NQP + j;                                                                      \
      if (q < QA) {                                                                                   \
        const int r = q * RPQ + lane / CH;                                                            \
        const int cc = (lane % CH) ^ swz<BK>(r);                                                      \
        const int row = gather ? grow[(ti) & 1][r] : t_r0 + min(r, t_rows - 1);                       \
        src[j] = A + (size_t)row * K + cc * 8;                                                        \
        ldsoff[j] = q * 512;                                                                          \
      } else {                                                                                        \
        const int nb = (q - QA) / QB, qq = (q - QA) % QB;                                             \
        const int r = qq * RPQ + lane / CH;                                                           \
        const int cc = (lane % CH) ^ swz<BK>(r);                                                      \
        src[j] = (nb == 0 ? B0 : B1) + ((size_t)t_e * N + min(t_n0 + r, N - 1)) * K + cc * 8;         \
        ldsoff[j] = A_ELEMS + nb * B_ELEMS + qq * 512;                                                \
      }                                                                                               \
    }                                                                                                 \
    if constexpr (F8) {                                                                               \
      const int srow = K / 16;                                                                        \
      _Pragma("unroll") for (int j = 0; j < NSP; ++j) {                                               \
        const int q = p * NSP + j;                                                                    \
        if (q < SQA) {                                                                                \
          const int r = q * 64 + lane;                                                                \
          const int row = gather ? grow[(ti) & 1][r] : t_r0 + min(r, t_rows - 1);                     \
          ssrc[j] = mx.a + (size_t)row * srow;                                                        \
          sldsoff[j] = (A_ELEMS + NB * B_ELEMS) * 2 + q * 256;                                        \
        } else {                                                                                      \
          const int nb = (q - SQA) / SQB, qq = (q - SQA) % SQB;                                       \
          const int r = qq * 64 + lane;                                                               \
          ssrc[j] = (nb == 0 ? mx.b0 : mx.b1) + ((size_t)t_e * N + min(t_n0 + r, N - 1)) * srow;      \
          sldsoff[j] = (A_ELEMS + NB * B_ELEMS) * 2 + BM * 4 + nb * BN * 4 + qq * 256;                \
        }                                                                                             \
      }                                                                                               \
    }                                                                                                 \
  }
#define MOE_WSP_ISSUE(slot)                                                                           \
  {                                                                                                   \
    const int base = (slot) * STAGE;                                                                  \
    _Pragma("unroll") for (int j = 0; j < NQP; ++j)                                                   \
      __builtin_amdgcn_global_load_lds((gas_ptr)(src[j] + ist * BK), (las_ptr)&lds[base + ldsoff[j]], 16, 0, 0); \
    if constexpr (F8) {                                                                               \
      _Pragma("unroll") for (int j = 0; j < NSP; ++j)                                                 \
        __builtin_amdgcn_global_load_lds((gas_ptr)(ssrc[j] + ist * 4),                                \
                                         (las_ptr)(reinterpret_cast<uint8_t*>(lds) + base * 2 + sldsoff[j]), 4, 0, 0); \
    }                                                                                                 \
    ++ist;                                                                                            \
  }
    int it = 0, ist = 0;  // tile and K-step of the next stage to issue
    int fslot = 0;        // its LDS ring slot
    bool more = true;     // whether tile `it` still has stages to issue
    MOE_WSP_SET_TILE(0)
    for (int f = 0; f < S - 1; ++f) {  // nsteps >= 4: both stages belong to the first tile
      MOE_WSP_ISSUE(fslot)
      fslot = fslot + 1 == S ? 0 : fslot + 1;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NQW));  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int ti = 0;; ++ti) {
      if (claimed[ti & 3] < 0) break;
      for (int st = 0; st < nsteps; ++st) {
        // the stage S-1 ahead: this tile's, or the first stages of the next claimed tile
        if (more && ist == nsteps) {
          const int tn = claimed[(it + 1) & 3];
          if (tn >= 0) {
            ++it;
            ist = 0;
            MOE_WSP_SET_TILE(it)
          } else {
            more = false;
          }
        }
        if (more) {
          MOE_WSP_ISSUE(fslot)
          fslot = fslot + 1 == S ? 0 : fslot + 1;
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(NQW));  // the stage consumed next has landed
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
#undef MOE_WSP_ISSUE
#undef MOE_WSP_SET_TILE
    return;
  }

  // ---------------- MFMA waves
  const int wm = wave / WN, wn = wave % WN;
  f32x4 acc[NB][FM][FN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[nb][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
  int aoffs[2][FM], boffs[2][FN];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = h * 4 + (lane >> 4);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int r = wm * TM + fm * 16 + (lane & 15);
      aoffs[h][fm] = r * BK + ((c ^ swz<BK>(r)) << 3);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int r = wn * TN + fn * 16 + (lane & 15);
      boffs[h][fn] = A_ELEMS + r * BK + ((c ^ swz<BK>(r)) << 3);
    }
  }
  struct Ops {
    bf16x8 a[FM];
    bf16x8 b[NB][FN];
  };
  constexpr int NR = FM + NB * FN, NM = NB * FN * FM;
  auto rd = [&](Ops& o, const uint16_t* base, int h) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) o.a[fm] = as_bf16x8(*reinterpret_cast<const u32x4*>(base + aoffs[h][fm]));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        o.b[nb][fn] = as_bf16x8(*reinterpret_cast<const u32x4*>(base + nb * B_ELEMS + boffs[h][fn]));
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[nb][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[fm], o.b[nb][fn], acc[nb][fm][fn], 0, 0, 0);
  };
  auto interleave = [] {
#pragma unroll
    for (int i = 0; i < (NR < NM ? NR : NM); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
  };
  // this wave's reads of the current stage are done; the loaders' next stage has landed
  auto barrier = [] {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto f8_step = [&](const uint16_t* base) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    constexpr int SCB = (A_ELEMS + NB * B_ELEMS) * 2;
    const int g = lane >> 4;
    const uint8_t* base8 = reinterpret_cast<const uint8_t*>(base);
    u32x4 a0[FM], a1[FM], b0[NB][FN], b1[NB][FN];
    int sa[FM], sb[NB][FN];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        b0[nb][fn] = *reinterpret_cast<const u32x4*>(base + nb * B_ELEMS + boffs[0][fn]);
        b1[nb][fn] = *reinterpret_cast<const u32x4*>(base + nb * B_ELEMS + boffs[1][fn]);
        sb[nb][fn] = base8[SCB + BM * 4 + nb * BN * 4 + (wn * TN + fn * 16 + (lane & 15)) * 4 + g];
      }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) sa[fm] = base8[SCB + (wm * TM + fm * 16 + (lane & 15)) * 4 + g];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      a0[fm] = *reinterpret_cast<const u32x4*>(base + aoffs[0][fm]);
      a1[fm] = *reinterpret_cast<const u32x4*>(base + aoffs[1][fm]);
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0[fm], a1[fm], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const i32x8 bv = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0[nb][fn], b1[nb][fn], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[nb][fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[nb][fm][fn], 0, 0, 0,
                                                                             sa[fm], 0, sb[nb][fn]);
        }
    }
  };

  Ops o0, o1;
  barrier();  // stage 0 has landed
  int cs = 0;  // ring slot of the stage the next K-step consumes
  auto next_slot = [](int x) { return x + 1 == S ? 0 : x + 1; };
  for (int ti = 0;; ++ti) {
    const int t = __builtin_amdgcn_readfirstlane(claimed[ti & 3]);
    if (t < 0) break;
    int t_e, t_r0, t_rows, t_n0;
    MOE_WSP_COORDS(centry[ti & 3], t_e, t_r0, t_rows, t_n0)
    (void)t_e;
    if (wm * TM >= t_rows) {  // no valid rows for this wave: keep the barrier cadence
      for (int st = 0; st < nsteps; ++st) {
        barrier();
        cs = next_slot(cs);
      }
      continue;
    }
    if constexpr (F8) {
      for (int st = 0; st < nsteps; ++st) {
        f8_step(lds + cs * STAGE);
        barrier();
        cs = next_slot(cs);
      }
    } else {
      // operands double-buffered in registers: the next 32-wide substep's LDS reads
      // are interleaved with the current substep's MFMAs
      rd(o0, lds + cs * STAGE, 0);
      for (int st = 0; st < nsteps - 1; ++st) {
        rd(o1, lds + cs * STAGE, 1);
        mma(o0);
        interleave();
        barrier();
        cs = next_slot(cs);
        rd(o0, lds + cs * STAGE, 0);
        mma(o1);
        interleave();
      }
      rd(o1, lds + cs * STAGE, 1);
      mma(o0);
      interleave();
      barrier();
      cs = next_slot(cs);
      mma(o1);
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * TM + fm * 16 + (lane >> 4) * 4 + i;
          const int c = t_n0 + wn * TN + fn * 16 + (lane & 15);
          if (r < t_rows && c < N)
            epi_store<EPI>(C, (size_t)(t_r0 + r) * N + c, acc[0][fm][fn][i],
                           NB > 1 ? acc[NB - 1][fm][fn][i] : 0.f, nullptr, c);
          acc[0][fm][fn][i] = 0.f;
          if constexpr (NB > 1) acc[NB - 1][fm][fn][i] = 0.f;
        }
  }
#undef MOE_WSP_COORDS
}

// ------------------------------------------------------------------ decode kernel
// For experts with a handful of rows: 16-row m-tiles, no LDS, every wave
// streams its own 16*FN weight rows straight from HBM with two K-steps of loads
// in flight.  bf16: within a 64-wide K-step lane l carries k = 16*(l/16) .. +16 of
// both operands (two 8-element MFMA halves); the same permutation of k on A and
// B leaves the sum unchanged and makes each weight row's 128 bytes one
// contiguous read by 4 lanes.  F8 (MXFP8 codes passed as 16-bit pairs, K = D / 2):
// a K-step is 128 codes, and lane l carries chunks g and 4 + g (g = l / 16) of it,
// the layout of v_mfma_scale_f32_16x16x128_f8f6f4, plus the E8M0 scales of block g
// of its A row and of each of its B rows.

template <int NB, int FN>
struct DecodeRegs {
  uint4 a[2];
  uint4 b[NB][FN][2];
  int sa;
  int sb[NB][FN];
};

template <int NB, int FN, bool F8>
__device__ __forceinline__ void decode_load(DecodeRegs<NB, FN>& r, const uint16_t* pa,
                                            const uint16_t* const (&pb)[NB][FN], int k0,
                                            const uint8_t* psa, const uint8_t* const (&psb)[NB][FN]) {
  constexpr int second = F8 ? 32 : 8;  // 16-bit offset of the lane's second chunk
  r.a[0] = *reinterpret_cast<const uint4*>(pa + k0);
  r.a[1] = *reinterpret_cast<const uint4*>(pa + k0 + second);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      r.b[nb][fn][0] = *reinterpret_cast<const uint4*>(pb[nb][fn] + k0);
      r.b[nb][fn][1] = *reinterpret_cast<const uint4*>(pb[nb][fn] + k0 + second);
    }
  if constexpr (F8) {
    const int s4 = k0 / 16;  // 4 scale bytes per 64-pair K-step
    r.sa = psa[s4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) r.sb[nb][fn] = psb[nb][fn][s4];
  }
}

template <int NB, int FN, bool F8>
__device__ __forceinline__ void decode_mma(f32x4 (&acc)[NB][FN], const DecodeRegs<NB, FN>& r) {
  if constexpr (F8) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(
        __builtin_bit_cast(u32x4, r.a[0]), __builtin_bit_cast(u32x4, r.a[1]), 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(
            __builtin_bit_cast(u32x4, r.b[nb][fn][0]), __builtin_bit_cast(u32x4, r.b[nb][fn][1]), 0, 1, 2, 3,
            4, 5, 6, 7));
        acc[nb][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[nb][fn], 0, 0, 0, r.sa, 0,
                                                                       r.sb[nb][fn]);
      }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 a = as_bf16x8(r.a[h]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[nb][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(r.b[nb][fn][h]),
                                                                 acc[nb][fn], 0, 0, 0);
    }
  }
}

template <int NB, int FN, int EPI, bool F8 = false>
__global__ __launch_bounds__(256) void k_gemm_decode(
    const uint16_t* __restrict__ A, int M, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ mtile_start, int E, int N, int K, const int32_t* __restrict__ gather,
    MxScales mx) {
  constexpr int BM = 16, BN = 4 * 16 * FN;
  TileCoord tc;
  if (!decode_tile<BM, BN>(offsets, mtile_start, E, M, N, tc)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int kl = F8 ? g * 8 : g * 16;
  // gather non-NULL: operand row r is A[gather[r]] (token rows read in permuted order)
  const int ar = tc.row0 + min(lane & 15, tc.rows - 1);
  const int arow = gather ? gather[ar] : ar;
  const uint16_t* pa = A + (size_t)arow * K + kl;
  const uint16_t* pb[NB][FN];
  const uint8_t* psa = nullptr;
  const uint8_t* psb[NB][FN];
  const int srow = K / 16;  // MXFP8 scale bytes per row
  if constexpr (F8) psa = mx.a + (size_t)arow * srow + g;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int gn = min(tc.n0 + wave * 16 * FN + fn * 16 + (lane & 15), N - 1);
    pb[0][fn] = B0 + ((size_t)tc.e * N + gn) * K + kl;
    if constexpr (NB > 1) pb[NB - 1][fn] = B1 + ((size_t)tc.e * N + gn) * K + kl;
    psb[0][fn] = nullptr;
    if constexpr (NB > 1) psb[NB - 1][fn] = nullptr;
    if constexpr (F8) {
      psb[0][fn] = mx.b0 + ((size_t)tc.e * N + gn) * srow + g;
      if constexpr (NB > 1) psb[NB - 1][fn] = mx.b1 + ((size_t)tc.e * N + gn) * srow + g;
    }
  }
  f32x4 acc[NB][FN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[nb][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  DecodeRegs<NB, FN> r0, r1;
  const int steps = K / 64;
  decode_load<NB, FN, F8>(r0, pa, pb, 0, psa, psb);
  if (steps > 1) decode_load<NB, FN, F8>(r1, pa, pb, 64, psa, psb);
  for (int s = 0; s < steps; s += 2) {
    decode_mma<NB, FN, F8>(acc, r0);
    if (s + 2 < steps) decode_load<NB, FN, F8>(r0, pa, pb, (s + 2) * 64, psa, psb);
    if (s + 1 < steps) {
      decode_mma<NB, FN, F8>(acc, r1);
      if (s + 3 < steps) decode_load<NB, FN, F8>(r1, pa, pb, (s + 3) * 64, psa, psb);
    }
  }
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (lane >> 4) * 4 + i;
      const int c = tc.n0 + wave * 16 * FN + fn * 16 + (lane & 15);
      if (r < tc.rows && c < N)
        epi_store<EPI>(C, (size_t)(tc.row0 + r) * N + c, acc[0][fn][i],
                       NB > 1 ? acc[NB - 1][fn][i] : 0.f, nullptr, c);
    }
}

// ------------------------------------------------------------------ decode down GEMM + combine
// Decode-scale steps: the expert down GEMM and the combine in one launch, with no
// hand-off of data between workgroups.  Workgroup b owns output columns
// [16 b, 16 b + 16) of EVERY row: its waves run the down GEMM's 16-row m-tiles of all
// touched experts for those 16 columns only (streaming each expert's 16 x K slice of
// W2 once), keep the bf16 Y columns of all R rows in LDS, and after one barrier the
// whole workgroup combines them: out[t, c] = sum_j w[t, j] * Y[token_row[t, j], c]
// (+ add[t, c]), fp32 fma in ascending j, one rounding, the bits k_combine produces.
// Each m-tile runs the K-steps, operand layout and MFMA sequence of k_gemm_decode (a
// lane carries k = 16 g .. 16 g + 15 of a 64-wide K-step, g = lane / 16), so Y has
// the bits of the separate down GEMM.  The waves keep DEPTH - 1 K-steps of loads in
// flight across m-tile boundaries; the m-tile table and segment starts are read from
// LDS.

constexpr int kDcCols = 16;  // output columns per workgroup

// LDS bytes of k_down_combine for E experts, R rows and at most `tiles` m-tiles:
// segment starts, m-tile table, token_row and routing weights, Y columns.
static inline size_t down_combine_lds(int E, int R, int tiles) {
  return ((size_t)(E + 1) + tiles + 2 * (size_t)R) * 4 + (size_t)R * kDcCols * 2;
}

template <int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void k_down_combine(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W2, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ mtile_start, int E, int N, int K, int R, const int32_t* __restrict__ token_row,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ add, int T, int k, void* __restrict__ out,
    int out_f32, uint16_t* __restrict__ y_out, int tiles_cap) {
  extern __shared__ __attribute__((aligned(16))) int32_t dc_lds[];
  int32_t* s_off = dc_lds;                          // [E + 1] segment starts
  int32_t* s_tile = s_off + (E + 1);                // [tiles] expert | m-tile << 16 of each m-tile
  int32_t* s_trow = s_tile + tiles_cap;             // [T * k] token_row
  float* s_w = reinterpret_cast<float*>(s_trow + R);  // [T * k] routing weights
  uint16_t* ys = reinterpret_cast<uint16_t*>(s_w + R);  // [R x 16] Y columns of every row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int total = mtile_start[E];
  for (int a = tid; a < T * k; a += NW * 64) {
    s_trow[a] = token_row[a];
    s_w[a] = topk_w[a];
  }
  for (int e = tid; e <= E; e += NW * 64) s_off[e] = offsets[e];
  for (int e = tid; e < E; e += NW * 64) {
    const int mt0 = mtile_start[e], mte = mtile_start[e + 1] - mt0;
    for (int m = 0; m < mte; ++m) s_tile[mt0 + m] = e | (m << 16);
  }
  __syncthreads();
  const int n0 = blockIdx.x * kDcCols;
  const int g = lane >> 4, c = lane & 15;
  const int my_tiles = total > wave ? ceil_div(total - wave, NW) : 0;  // tiles wave + NW q
  const int S = K / 64;

  // Issue side: tile i_q, K-step i_s.  Every K-step issues the same loads (past the
  // wave's last tile they re-read that tile's last step: valid addresses, results
  // unused), so the compiler's load-count waits stay exact and DEPTH - 1 steps stay in
  // flight across tile boundaries.
  int i_q = 0, i_s = 0;
  const uint16_t* ipa = A;
  const uint16_t* ipb[1][1] = {{W2}};
  const uint8_t* const no_scale[1][1] = {{nullptr}};
  auto issue = [&](DecodeRegs<1, 1>& r) {
    if (i_s == 0 && i_q < my_tiles) {
      const int v = s_tile[wave + i_q * NW];
      const int e = v & 0xffff;
      const int row0 = s_off[e] + (v >> 16) * 16;
      const int rows = min(16, s_off[e + 1] - row0);
      ipa = A + (size_t)(row0 + min(c, rows - 1)) * K + g * 16;
      ipb[0][0] = W2 + ((size_t)e * N + n0 + c) * K + g * 16;
    }
    decode_load<1, 1, false>(r, ipa, ipb, min(i_s, S - 1) * 64, nullptr, no_scale);
    if (i_q < my_tiles && ++i_s == S) {
      i_s = 0;
      ++i_q;
    }
  };
  if (my_tiles > 0) {
    DecodeRegs<1, 1> ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue(ring[d]);
    for (int q = 0; q < my_tiles; ++q) {
      f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
      for (int s0 = 0; s0 < S; s0 += DEPTH) {  // DEPTH divides S
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          issue(ring[(d + DEPTH - 1) % DEPTH]);
          decode_mma<1, 1, false>(acc, ring[d]);
        }
      }
      // m-tile done: its 16 x 16 Y block, rounded to bf16, into LDS
      const int v = s_tile[wave + q * NW];
      const int e = v & 0xffff;
      const int row0 = s_off[e] + (v >> 16) * 16;
      const int rows = min(16, s_off[e + 1] - row0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        if (r < rows) {
          const uint16_t y = f32_to_bf16(acc[0][0][i]);
          ys[(row0 + r) * kDcCols + c] = y;
          if (y_out) y_out[(size_t)(row0 + r) * N + n0 + c] = y;
        }
      }
    }
  }
  __syncthreads();
  // combine of this workgroup's 16 columns for every token
  for (int idx = tid; idx < T * kDcCols; idx += NW * 64) {
    const int t = idx / kDcCols, cc = idx % kDcCols;
    float a = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = s_trow[t * k + j];
      if (r < 0) continue;  // dropped by an expert capacity: no term
      a = fmaf(s_w[t * k + j], bf16_to_f32(ys[r * kDcCols + cc]), a);
    }
    const size_t o = (size_t)t * N + n0 + cc;
    if (add) a += bf16_to_f32(add[o]);
    if (out_f32) static_cast<float*>(out)[o] = a;
    else static_cast<uint16_t*>(out)[o] = f32_to_bf16(a);
  }
}

// ------------------------------------------------------------------ fp32 SIMT kernel
// fp32 layers and the exact-input fp32 gate: 64x64 tile, 16x16 threads with
// 4x4 outputs each, K chunks of 16 through LDS; each output is one fma chain
// over ascending k.  A is fp32 or bf16 (widened exactly), B is fp32.

constexpr int kSBK = 16;

template <typename AT>
__device__ __forceinline__ float load_as_f32(const AT* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename AT, int NB, int EPI>
__global__ __launch_bounds__(256) void k_gemm_simt(const AT* __restrict__ A, int M,
                                                   const float* __restrict__ B0,
                                                   const float* __restrict__ B1,
                                                   void* __restrict__ C,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ mtile_start, int E,
                                                   int N, int K, const float* __restrict__ bias) {
  constexpr int BM = 64, BN = 64;
  __shared__ float sA[kSBK][BM + 4];
  __shared__ float sB[NB][kSBK][BN + 4];
  TileCoord tc;
  if (!decode_tile<BM, BN>(offsets, mtile_start, E, M, N, tc)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* Bm[2] = {B0 + (size_t)tc.e * N * K, NB > 1 ? B1 + (size_t)tc.e * N * K : nullptr};
  float acc[NB][4][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nb][i][j] = 0.f;
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row lr, k lk .. lk+3
  for (int k0 = 0; k0 < K; k0 += kSBK) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = k0 + lk + q;
      float va = 0.f;
      if (lr < tc.rows && kk < K) va = load_as_f32<AT>(A + (size_t)(tc.row0 + lr) * K + kk);
      sA[lk + q][lr] = va;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float vb = 0.f;
        if (tc.n0 + lr < N && kk < K) vb = Bm[nb][(size_t)(tc.n0 + lr) * K + kk];
        sB[nb][lk + q][lr] = vb;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSBK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty + 16 * i];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = sB[nb][kk][tx + 16 * j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nb][i][j] = fmaf(a[i], b, acc[nb][i][j]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ty + 16 * i, c = tc.n0 + tx + 16 * j;
      if (r < tc.rows && c < N)
        epi_store<EPI>(C, (size_t)(tc.row0 + r) * N + c, acc[0][i][j],
                       NB > 1 ? acc[NB - 1][i][j] : 0.f, bias, c);
    }
}

// ------------------------------------------------------------------ launchers

static inline int grid_for(int max_mtiles, int N, int BN) {
  const long tiles = (long)max_mtiles * ceil_div(N, BN);
  return (int)(ceil_div((int)tiles, 8) * 8);
}

int gemm_bm(GemmKind kind) {
  switch (kind) {
    case GEMM_PREFILL: return 128;
    case GEMM_DECODE: return 16;
    default: return 64;
  }
}

int max_mtiles(int M, int E, int bm) {
  // sum_e ceil(n_e / bm) <= floor(M / bm) + (number of non-empty experts)
  return M / bm + (E < M ? E : M) + 1;
}

// Kernel per GEMM, measured on MI355X with the real per-expert row counts of the
// Qwen3-30B-A3B-shaped, DeepSeek-R1-shaped and latent layers (one box, one run):
//  - expert gate/up: the persistent wave-specialised LDS-DMA kernel, 128 x 128
//    tiles, 8 MFMA waves (against one workgroup per tile: Qwen3-shaped 303 -> 271 us,
//    R1-shaped 4.66 -> 4.45 ms, latent equal; against 256-row tiles with every wave
//    loading, faster on both of the first two); one workgroup per tile (n-tiles in
//    pairs from 16 n-tiles on) when the persistent kernel's tile table does not fit;
//  - expert down: the persistent wave-specialised kernel.  128 x 256 tiles (half
//    the re-reads of the intermediate rows) when K < 2048 or the experts average
//    at least 192 rows: Qwen3-shaped (K = 768, 256 rows) 174 us against 189 us for
//    the register-staged kernel at three waves per SIMD and 187 / 208 us for
//    256 x 128 / 128 x 128 persistent tiles; R1-shaped (K = 2048, 256 rows) 2.30 ms
//    against 2.61 ms on 256 x 128 tiles.  Otherwise 256 x 128 tiles for K >= 2048
//    (latent-shaped, 128 rows: 0.89 ms against 0.94 ms on 128 x 256 tiles; R1-shaped
//    2.61 -> 2.46 ms against one workgroup per tile), and the register-staged
//    kernel when no persistent tile table fits;
//  - dense latent projections (one group): wave-specialised kernel with
//    256 x 128 tiles (one tile row per 256 tokens fills 256 CUs in one pass).
GemmChoice choose_gemm(GemmKind kind, bool swiglu, bool grouped, bool f8, int M, int E, int N, int K) {
  if (kind == GEMM_SIMT)
    return {GV_SIMT, 64, 64, false, swiglu ? "k_gemm_simt<float, 2," : "k_gemm_simt<float, 1,"};
  if (kind == GEMM_DECODE) {
    if (swiglu) return {f8 ? GV_DECODE_SWIGLU_F8 : GV_DECODE_SWIGLU, 16, 128, false, "k_gemm_decode<2, 2,"};
    return {GV_DECODE, 16, 128, false, "k_gemm_decode<1, 2,"};
  }
  if (!grouped) return {GV_WS_256x128, 256, 128, false, "k_gemm_ws<256, 128, 1,"};
  if (swiglu) {
    const long tiles = (long)max_mtiles(M, E, 128) * ceil_div(N, 128);
    const bool fits = f8 ? wsp_fits<true>(tiles, M, 128, E, N, K) : wsp_fits<false>(tiles, M, 128, E, N, K);
    if (fits) return {f8 ? GV_WSP_128x128_SWIGLU_F8 : GV_WSP_128x128_SWIGLU, 128, 128, true, "k_gemm_wsp<128, 128, 2,"};
    if (ceil_div(N, 128) >= 16)
      return {f8 ? GV_WS_128x128_SWIGLU_PAIRS_F8 : GV_WS_128x128_SWIGLU_PAIRS, 128, 128, false, "k_gemm_ws<128, 128, 2,"};
    return {f8 ? GV_WS_128x128_SWIGLU_F8 : GV_WS_128x128_SWIGLU, 128, 128, false, "k_gemm_ws<128, 128, 2,"};
  }
  if (f8) return {GV_NONE, 0, 0, false, "none"};  // MXFP8 operands feed the gate/up GEMM only
  if (K < 2048 || (long)M >= 192L * E) {
    const long tiles = (long)max_mtiles(M, E, 128) * ceil_div(N, 256);
    if (wsp_fits<false>(tiles, M, 128, E, N, K)) return {GV_WSP_128x256, 128, 256, true, "k_gemm_wsp<128, 256, 1,"};
  }
  if (K >= 2048) {
    const long tiles = (long)max_mtiles(M, E, 256) * ceil_div(N, 128);
    if (wsp_fits<false>(tiles, M, 256, E, N, K)) return {GV_WSP_256x128, 256, 128, true, "k_gemm_wsp<256, 128, 1,"};
    return {GV_WS_256x128, 256, 128, false, "k_gemm_ws<256, 128, 1,"};
  }
  return {GV_PREFILL_128x128, 128, 128, false, "k_gemm_prefill<128, 128, 1,"};
}

bool gemm_gather_ok(int M, int E, int N, int K, bool mx) {
  return choose_gemm(GEMM_PREFILL, true, true, mx, M, E, N, K).persistent;
}

// The persistent kernels' claim counters: slots 0-7 for the gate/up GEMM, 8-15 for the
// down GEMM, after the two m-tile tables.
static inline int32_t* claim_slots(const int32_t* mtile_start, int E, bool down) {
  return const_cast<int32_t*>(mtile_start) + 2 * (E + 1) + (down ? 8 : 0);
}

#define MOE_WSP(BM_, BN_, NB_, EPI_, F8_, a_, b0_, b1_, mt_, mx_, gather_)                                   \
  hipLaunchKernelGGL((k_gemm_wsp<BM_, BN_, NB_, EPI_, 3, 8, F8_>), dim3(256), dim3(8 * 64 + 192), 0, st, a_, \
                     M, b0_, b1_, C, offsets, mt_, E, N, K, mx_, claim_slots(mtile_start, E, NB_ == 1),    \
                     gather_)
#define MOE_WS(BM_, G_, NB_, EPI_, F8_, a_, b0_, b1_, mt_, grid_, mx_)                                        \
  hipLaunchKernelGGL((k_gemm_ws<BM_, 128, NB_, EPI_, 3, 8, 64, G_, F8_>), dim3(grid_), dim3(8 * 64 + 128), 0,  \
                     st, a_, M, b0_, b1_, C, offsets, mt_, E, N, K, mx_)
#define MOE_DEC(NB_, EPI_, F8_, a_, b0_, b1_, gather_, mx_)                                                 \
  hipLaunchKernelGGL((k_gemm_decode<NB_, 2, EPI_, F8_>), dim3(grid_for(max_mtiles(M, E, 16), N, 128)),       \
                     dim3(256), 0, st, a_, M, b0_, b1_, C, offsets, mtile_start, E, N, K, gather_, mx_)

hipError_t launch_gemm_prefill_gather(int epi, const uint16_t* X, const int32_t* gather, int M,
                                      const uint16_t* B0, const uint16_t* B1, void* C,
                                      const int32_t* offsets, const int32_t* mtile_start, int E, int N,
                                      int K, hipStream_t st) {
  if (!gather || !gemm_gather_ok(M, E, N, K, false)) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU_BF16)
    MOE_WSP(128, 128, 2, EPI_SWIGLU_BF16, false, X, B0, B1, mtile_start, MxScales{}, gather);
  else if (epi == EPI_SWIGLU_F32)
    MOE_WSP(128, 128, 2, EPI_SWIGLU_F32, false, X, B0, B1, mtile_start, MxScales{}, gather);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(GemmKind kind, int epi, const uint16_t* A, int M, const uint16_t* B0,
                            const uint16_t* B1, void* C, const int32_t* offsets,
                            const int32_t* mtile_start, int E, int N, int K, hipStream_t st) {
  const bool swiglu = epi == EPI_SWIGLU_BF16 || epi == EPI_SWIGLU_F32;
  if (kind == GEMM_SIMT || (!offsets && swiglu)) return hipErrorInvalidValue;
  if (swiglu ? !(epi == EPI_SWIGLU_BF16 || epi == EPI_SWIGLU_F32) : !(epi == EPI_BF16 || epi == EPI_F32))
    return hipErrorInvalidValue;
  const GemmChoice c = choose_gemm(kind, swiglu, offsets != nullptr, false, M, E, N, K);
  const int32_t* no_gather = nullptr;
  const int32_t* mt256 = offsets ? mtile_start + E + 1 : nullptr;  // second m-tile table (256-row tiles)
  const bool f32 = epi == EPI_F32 || epi == EPI_SWIGLU_F32;
  switch (c.v) {
    case GV_WSP_128x128_SWIGLU:
      if (f32) MOE_WSP(128, 128, 2, EPI_SWIGLU_F32, false, A, B0, B1, mtile_start, MxScales{}, no_gather);
      else MOE_WSP(128, 128, 2, EPI_SWIGLU_BF16, false, A, B0, B1, mtile_start, MxScales{}, no_gather);
      break;
    case GV_WS_128x128_SWIGLU_PAIRS: {
      const int g = grid_for(max_mtiles(M, E, 128), N, 128);
      if (f32) MOE_WS(128, 2, 2, EPI_SWIGLU_F32, false, A, B0, B1, mtile_start, g, MxScales{});
      else MOE_WS(128, 2, 2, EPI_SWIGLU_BF16, false, A, B0, B1, mtile_start, g, MxScales{});
      break;
    }
    case GV_WS_128x128_SWIGLU: {
      const int g = grid_for(max_mtiles(M, E, 128), N, 128);
      if (f32) MOE_WS(128, 1, 2, EPI_SWIGLU_F32, false, A, B0, B1, mtile_start, g, MxScales{});
      else MOE_WS(128, 1, 2, EPI_SWIGLU_BF16, false, A, B0, B1, mtile_start, g, MxScales{});
      break;
    }
    case GV_WSP_128x256:
      if (f32) MOE_WSP(128, 256, 1, EPI_F32, false, A, B0, B1, mtile_start, MxScales{}, no_gather);
      else MOE_WSP(128, 256, 1, EPI_BF16, false, A, B0, B1, mtile_start, MxScales{}, no_gather);
      break;
    case GV_WSP_256x128:
      if (f32) MOE_WSP(256, 128, 1, EPI_F32, false, A, B0, B1, mt256, MxScales{}, no_gather);
      else MOE_WSP(256, 128, 1, EPI_BF16, false, A, B0, B1, mt256, MxScales{}, no_gather);
      break;
    case GV_WS_256x128: {
      // grouped: 256-row tiles on the second m-tile table; dense: one group of M rows
      const int g = grid_for(offsets ? max_mtiles(M, E, 256) : ceil_div(M, 256), N, 128);
      if (f32) MOE_WS(256, 1, 1, EPI_F32, false, A, B0, B1, mt256, g, MxScales{});
      else MOE_WS(256, 1, 1, EPI_BF16, false, A, B0, B1, mt256, g, MxScales{});
      break;
    }
    case GV_PREFILL_128x128: {
      const dim3 g(grid_for(max_mtiles(M, E, 128), N, 128));
      if (f32)
        hipLaunchKernelGGL((k_gemm_prefill<128, 128, 1, EPI_F32, 3>), g, dim3(256), 0, st, A, M, B0, B1, C,
                           offsets, mtile_start, E, N, K);
      else
        hipLaunchKernelGGL((k_gemm_prefill<128, 128, 1, EPI_BF16, 3>), g, dim3(256), 0, st, A, M, B0, B1, C,
                           offsets, mtile_start, E, N, K);
      break;
    }
    case GV_DECODE_SWIGLU:
      if (f32) MOE_DEC(2, EPI_SWIGLU_F32, false, A, B0, B1, no_gather, MxScales{});
      else MOE_DEC(2, EPI_SWIGLU_BF16, false, A, B0, B1, no_gather, MxScales{});
      break;
    case GV_DECODE:
      if (f32) MOE_DEC(1, EPI_F32, false, A, B0, B1, no_gather, MxScales{});
      else MOE_DEC(1, EPI_BF16, false, A, B0, B1, no_gather, MxScales{});
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_simt(bool a_bf16, int epi, const void* A, int M, const float* B0,
                            const float* B1, void* C, const int32_t* offsets,
                            const int32_t* mtile_start, int E, int N, int K, const float* bias,
                            hipStream_t st) {
  const int mt = offsets ? max_mtiles(M, E, 64) : ceil_div(M, 64);
  const int g = grid_for(mt, N, 64);
#define MOE_SIMT(AT, NB, EP)                                                                   \
  hipLaunchKernelGGL((k_gemm_simt<AT, NB, EP>), dim3(g), dim3(256), 0, st,                     \
                     static_cast<const AT*>(A), M, B0, B1, C, offsets, mtile_start, E, N, K, bias)
  if (a_bf16) {
    switch (epi) {
      case EPI_F32_BIAS: MOE_SIMT(uint16_t, 1, EPI_F32_BIAS); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      case EPI_F32_BIAS: MOE_SIMT(float, 1, EPI_F32_BIAS); break;
      case EPI_F32: MOE_SIMT(float, 1, EPI_F32); break;
      case EPI_SWIGLU_F32: MOE_SIMT(float, 2, EPI_SWIGLU_F32); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_SIMT
  return hipGetLastError();
}

bool down_combine_ok(int R, int E, int N, int K) {
  return N % kDcCols == 0 && K % 64 == 0 && E < 65536 &&
         down_combine_lds(E, R, max_mtiles(R, E, 16)) <= kDownCombineMaxLds;
}

hipError_t launch_down_combine(const uint16_t* act, int R, const uint16_t* W2, const int32_t* offsets,
                               const int32_t* mtile_start, int E, int N, int K, const int32_t* token_row,
                               const float* topk_w, const void* add, int T, int k, void* out, bool out_f32,
                               void* y_out, hipStream_t st) {
  if (!down_combine_ok(R, E, N, K)) return hipErrorInvalidValue;
  const int tiles_cap = max_mtiles(R, E, 16);
  const size_t lds = down_combine_lds(E, R, tiles_cap);
  const int S = K / 64;  // K-steps per m-tile; the load pipeline's depth divides it
#define MOE_DC(DEPTH_)                                                                                      \
  hipLaunchKernelGGL((k_down_combine<16, DEPTH_>), dim3(N / kDcCols), dim3(16 * 64), lds, st, act, W2,      \
                     offsets, mtile_start, E, N, K, R, token_row, topk_w, static_cast<const uint16_t*>(add), \
                     T, k, out, (int)out_f32, static_cast<uint16_t*>(y_out), tiles_cap)
  if (S % 4 == 0) MOE_DC(4);
  else if (S % 2 == 0) MOE_DC(2);
  else MOE_DC(1);
#undef MOE_DC
  return hipGetLastError();
}

hipError_t launch_gemm_decode_gather(int epi, const uint16_t* X, const int32_t* gather, int M,
                                     const uint16_t* B0, const uint16_t* B1, void* C,
                                     const int32_t* offsets, const int32_t* mtile_start, int E, int N,
                                     int K, hipStream_t st) {
  if (epi != EPI_SWIGLU_BF16) return hipErrorInvalidValue;
  MOE_DEC(2, EPI_SWIGLU_BF16, false, X, B0, B1, gather, MxScales{});
  return hipGetLastError();
}

hipError_t launch_gemm_mx_swiglu(GemmKind kind, const uint8_t* A, int M, const uint8_t* B0, const uint8_t* B1,
                                 uint16_t* C, const int32_t* offsets, const int32_t* mtile_start, int E,
                                 int N, int D, MxScales mx, const int32_t* gather, hipStream_t st) {
  if (D % 128 || (kind != GEMM_PREFILL && kind != GEMM_DECODE)) return hipErrorInvalidValue;
  const uint16_t* a = reinterpret_cast<const uint16_t*>(A);
  const uint16_t* b0 = reinterpret_cast<const uint16_t*>(B0);
  const uint16_t* b1 = reinterpret_cast<const uint16_t*>(B1);
  const int K = D / 2;  // codes travel as 16-bit pairs
  const GemmChoice c = choose_gemm(kind, true, true, true, M, E, N, K);
  if (gather && kind == GEMM_PREFILL && !c.persistent) return hipErrorInvalidValue;
  switch (c.v) {
    case GV_WSP_128x128_SWIGLU_F8:
      MOE_WSP(128, 128, 2, EPI_SWIGLU_BF16, true, a, b0, b1, mtile_start, mx, gather);
      break;
    case GV_WS_128x128_SWIGLU_PAIRS_F8:
      MOE_WS(128, 2, 2, EPI_SWIGLU_BF16, true, a, b0, b1, mtile_start, grid_for(max_mtiles(M, E, 128), N, 128), mx);
      break;
    case GV_WS_128x128_SWIGLU_F8:
      MOE_WS(128, 1, 2, EPI_SWIGLU_BF16, true, a, b0, b1, mtile_start, grid_for(max_mtiles(M, E, 128), N, 128), mx);
      break;
    case GV_DECODE_SWIGLU_F8:
      MOE_DEC(2, EPI_SWIGLU_BF16, true, a, b0, b1, gather, mx);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#undef MOE_WSP
#undef MOE_WS
#undef MOE_DEC

}  // namespace moe
