// Internal launchers of the libmoe kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

enum Epi {
  EPI_BF16 = 0,         // C = bf16(acc)
  EPI_SWIGLU_BF16 = 1,  // C = bf16(SiLU(acc0) * acc1)
  EPI_F32 = 2,          // C = acc
  EPI_SWIGLU_F32 = 3,   // C = SiLU(acc0) * acc1
  EPI_F32_BIAS = 4      // C = acc + bias[col]
};

enum GemmKind { GEMM_PREFILL = 0, GEMM_DECODE = 1, GEMM_SIMT = 2 };

// An m-tile table buffer holds the tables for two tile heights, (E + 1) ints each,
// followed by kClaimSlots tile-claim counters of the persistent expert GEMMs (one per
// XCD for the gate/up GEMM, then one per XCD for the down GEMM), which the kernels
// that write the tables set to zero.
constexpr int kClaimSlots = 16;
inline size_t mtile_table_bytes(int E) { return ((size_t)(E + 1) * 2 + kClaimSlots) * 4; }

// E8M0 scale arrays of MXFP8 GEMM operands ([rows x K/32] bytes; NULL for bf16 GEMMs).
struct MxScales {
  const uint8_t* a;
  const uint8_t* b0;
  const uint8_t* b1;
};

// The kernel (and tile shape) one GEMM runs on; choose_gemm is the single place that
// decides it, for the launchers and for the host-side plan query alike.
enum GemmVariant {
  GV_NONE = 0,
  GV_WSP_128x128_SWIGLU,           // persistent, gate/up
  GV_WS_128x128_SWIGLU_PAIRS,      // one workgroup per tile, n-tiles in pairs
  GV_WS_128x128_SWIGLU,            // one workgroup per tile
  GV_WSP_128x256,                  // persistent, down
  GV_WSP_256x128,                  // persistent, down with a long K (256-row m-tile table)
  GV_WS_256x128,                   // one workgroup per tile, long-K down or dense projection
  GV_PREFILL_128x128,              // register-staged, down
  GV_DECODE_SWIGLU,                // 16-row tiles, gate/up
  GV_DECODE,                       // 16-row tiles, down
  GV_SIMT,                         // fp32
  GV_WSP_128x128_SWIGLU_F8,        // MXFP8 gate/up variants of the above
  GV_WS_128x128_SWIGLU_PAIRS_F8,
  GV_WS_128x128_SWIGLU_F8,
  GV_DECODE_SWIGLU_F8,
  GV_DOWN_COMBINE                  // decode-scale down GEMM fused with the combine
};
struct GemmChoice {
  GemmVariant v;
  int bm, bn;          // workgroup tile
  bool persistent;     // one workgroup per CU claiming tiles
  const char* kernel;  // the kernel's name up to its tile arguments, as a trace prints it
};
// swiglu: the gate/up GEMM (two weight matrices); grouped: per-expert row groups (else one
// dense group of M rows); f8: MXFP8 operands (K counts 16-bit code pairs).
GemmChoice choose_gemm(GemmKind kind, bool swiglu, bool grouped, bool f8, int M, int E, int N, int K);

int gemm_bm(GemmKind kind);
int max_mtiles(int M, int E, int bm);

// Where the top-k kernels read each token's E scores: a scores row [T x E], plus an
// optional bias added on the fly; or, with parts non-NULL, the gate's S split-K partial
// rows (slice p at parts + p * stride) summed in ascending p, plus the bias, and that
// sum also written to logits_out (the same bits k_gate_reduce would write).
struct ScoreSrc {
  const float* scores;
  const float* parts;
  int S;
  size_t stride;
  const float* bias;
  float* logits_out;
};
hipError_t launch_topk(const ScoreSrc& src, int T, int E, int k, int32_t* ids, float* w,
                       int32_t* block_counts, hipStream_t st);
hipError_t launch_block_counts(const int32_t* ids, int T, int E, int k, int32_t* block_counts,
                               hipStream_t st);
// block_counts[b][e] -> rows of e in blocks before b; counts_out[e] = total (if non-NULL).
// cap > 0: counts_out[e] = min(total, cap) (expert capacity; later assignments are dropped).
hipError_t launch_expert_scan(int32_t* block_counts, int nb, int E, int cap, int32_t* counts_out,
                              hipStream_t st);
// offsets_out from counts (if non-NULL) and, for bm > 0, the m-tile tables for tile heights
// bm and 2 bm; with offsets_in the counts are its differences.
hipError_t launch_offsets(const int32_t* counts, const int32_t* offsets_in, int E,
                          int32_t* offsets_out, int bm, int32_t* mtile_start, hipStream_t st);
// bases: per-block rows before each block (launch_expert_scan); offsets: segment starts.
// x_scale non-NULL: MXFP8 dispatch of bf16 rows (x_perm gets E4M3 codes, x_scale the
// [rows x D/32] E8M0 scales; row16 = D / 8 must be a multiple of 4).
// po (optional, fused layer): the permutation takes the segment starts from the
// per-expert counts itself (each workgroup scans them in LDS; `offsets` is then
// unused), and workgroup (0, 0) writes what launch_offsets(counts, NULL, E,
// po->offsets_out, po->bm, po->mtile_start) would, claim counters included, so the
// layer saves that launch.
struct PermuteOffsets {
  const int32_t* counts;
  int32_t* offsets_out;
  int bm;
  int32_t* mtile_start;
};
hipError_t launch_permute(const void* x, int row16, const int32_t* ids, int T, int E, int k, int cap,
                          const int32_t* offsets, const int32_t* bases, void* x_perm, uint8_t* x_scale,
                          int32_t* row_token, int32_t* token_row, hipStream_t st,
                          const PermuteOffsets* po = nullptr);
// MXFP8 quantisation of [rows x cols] bf16 or fp32 values (cols % 32 == 0).
hipError_t launch_mx_quantize(const void* src, bool src_bf16, long rows, long cols, uint8_t* q,
                              uint8_t* scale, hipStream_t st);
// Expert gate/up GEMM on MXFP8 rows and weights (D % 128 == 0), bf16 SwiGLU output;
// GEMM_DECODE may read its rows through gather (as launch_gemm_decode_gather), and so
// may GEMM_PREFILL when gemm_gather_ok(M, E, N, D / 2, true).
hipError_t launch_gemm_mx_swiglu(GemmKind kind, const uint8_t* A, int M, const uint8_t* B0, const uint8_t* B1,
                                 uint16_t* C, const int32_t* offsets, const int32_t* mtile_start, int E,
                                 int N, int D, MxScales mx, const int32_t* gather, hipStream_t st);
// add: nullable [T x row16 x 16 B] addend of the input element type, added after the k terms.
hipError_t launch_combine(const void* y, int row16, bool in_bf16, const int32_t* token_row,
                          const float* w, const void* add, int T, int k, void* out, bool out_f32,
                          hipStream_t st);
// dst[a] = src[index[a]] for a < min(R, *limit) (limit nullable), index < 0 skipped.
hipError_t launch_unpermute(const void* y, int row16, const int32_t* token_row, int R,
                            const int32_t* limit, void* y_tok, hipStream_t st);
hipError_t launch_weighted_reduce(const void* y_tok, int row16, bool in_bf16, const int32_t* token_row,
                                  const float* w, const void* add, int T, int k, void* out,
                                  bool out_f32, hipStream_t st);
// Decode-scale routing (T <= kSmallT) in one launch: ids, weights, counts, offsets, the m-tile
// tables (bm > 0) and row_token / token_row, as the large-T kernels produce them.  In one
// workgroup where route_one_workgroup(T, E, k), else over ceil(T / kMultiTok) workgroups that
// hand over through one 64-bit word of workspace (handover) with tag, a value in
// [1, 2^56) that no earlier call used.
hipError_t launch_route_small(const ScoreSrc& src, int T, int E, int k, int32_t* ids,
                             float* w, int32_t* counts, int32_t* offsets, int32_t* row_token,
                             int32_t* token_row, int cap, int bm, int32_t* mtile_start,
                             unsigned long long* handover, unsigned long long tag, hipStream_t st);
// Decode GEMM whose A rows are read through an index: row r of the operand is X[gather[r]]
// (the expert gate/up GEMM reading the token rows directly instead of a permuted copy).
// Whether the persistent prefill gate/up GEMM can read its rows through a gather
// index (row r of the grouped GEMM = row gather[r] of X): the tile table fits and K
// (16-bit columns; MXFP8 codes count in pairs) has at least 4 K-steps.
bool gemm_gather_ok(int M, int E, int N, int K, bool mx);
// Prefill gate/up GEMM (SwiGLU epilogue) on rows gathered from X through `gather`
// (row_token); requires gemm_gather_ok(M, E, N, K, false).
hipError_t launch_gemm_prefill_gather(int epi, const uint16_t* X, const int32_t* gather, int M,
                                      const uint16_t* B0, const uint16_t* B1, void* C,
                                      const int32_t* offsets, const int32_t* mtile_start, int E, int N,
                                      int K, hipStream_t st);
hipError_t launch_gemm_decode_gather(int epi, const uint16_t* X, const int32_t* gather, int M,
                                     const uint16_t* B0, const uint16_t* B1, void* C,
                                     const int32_t* offsets, const int32_t* mtile_start, int E, int N,
                                     int K, hipStream_t st);
// Decode-scale down GEMM fused with the combine (16-row m-tiles on the tables for
// tile height 16): out = combine(bf16(act W2^T)) with the bits of launch_gemm_bf16
// (GEMM_DECODE, EPI_BF16) followed by launch_combine; y_out (nullable) also receives
// Y [R x N].  Needs down_combine_ok(R, E, N, K): N % 16 == 0, K % 64 == 0 and the Y
// columns of all R rows plus the tile table in kDownCombineMaxLds bytes of LDS.
constexpr size_t kDownCombineMaxLds = 128 * 1024;
bool down_combine_ok(int R, int E, int N, int K);
hipError_t launch_down_combine(const uint16_t* act, int R, const uint16_t* W2, const int32_t* offsets,
                               const int32_t* mtile_start, int E, int N, int K, const int32_t* token_row,
                               const float* topk_w, const void* add, int T, int k, void* out, bool out_f32,
                               void* y_out, hipStream_t st);
// One group of T rows: offsets = {0, T} and the m-tile tables (tile heights bm, 2 bm) for E = 1.
hipError_t launch_single_group(int T, int32_t* offsets, int bm, int32_t* mtile_start, hipStream_t st);
// bf16 MFMA GEMM: C[r, n] = epi(sum_k A[r, k] * B[e(r)][n, k]); offsets == NULL means one dense group of M rows.
// mtile_start holds the m-tile tables for tile heights gemm_bm(kind) and 2 * gemm_bm(kind)
// (E + 1 entries each, as written by launch_offsets).
hipError_t launch_gemm_bf16(GemmKind kind, int epi, const uint16_t* A, int M, const uint16_t* B0,
                            const uint16_t* B1, void* C, const int32_t* offsets,
                            const int32_t* mtile_start, int E, int N, int K, hipStream_t st);
// Router logits = X gate_w^T + bias, X bf16, gate_w fp32 (split-bf16 MFMA, fp32 accuracy); H % 64 == 0.
// The gate kernel's tile width (32 or 64 experts per wave) and split-K count for a shape.
struct GatePlan {
  int tn, splits;
};
GatePlan gate_plan(int T, int E, int H);
// partial: gate_plan(T, E, H).splits * T * E floats of scratch (unused when that is 1).
// *splits (nullable) receives that count.  With defer_reduce and more than one slice the
// slices stay in partial and logits are written by the top-k kernel (ScoreSrc.parts).
hipError_t launch_gate_bf16(const uint16_t* x, const float* gate_w, const float* bias, float* logits,
                            float* partial, int T, int E, int H, hipStream_t st, bool defer_reduce,
                            int* splits);
// fp32 SIMT GEMM (A fp32 or bf16, B fp32).
hipError_t launch_gemm_simt(bool a_bf16, int epi, const void* A, int M, const float* B0,
                            const float* B1, void* C, const int32_t* offsets,
                            const int32_t* mtile_start, int E, int N, int K, const float* bias,
                            hipStream_t st);

}  // namespace moe
