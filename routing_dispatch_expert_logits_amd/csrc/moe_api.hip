// Host side of the libmoe C ABI: argument validation, workspace carve-up,
// kernel selection by shape, and the launch sequence of each call.  No call
// allocates, synchronises or reads device memory.
#include <atomic>
#include <climits>
#include <cstddef>
#include <cstdint>

#include "moe.h"
#include "moe_kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Carve {
  size_t cur = 0;
  size_t take(size_t bytes) {
    const size_t o = cur;
    cur = align_up(cur + bytes);
    return o;
  }
};

bool al16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al16_or_null(const void* p) { return !p || al16(p); }

struct Dims {
  int T, H, E, k, I, L, D, R, nb, es;
  int Is;   // shared expert intermediate width, 0 = none
  int cap;  // rows kept per expert, 0 = no limit
  bool bf16;
  bool mx;  // MXFP8 dispatch: x_perm holds E4M3 codes + E8M0 scales, W1 / W3 likewise
};

moe_status check_shape(const moe_shape* s, Dims& d) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 1 || s->H < 1 || s->E < 1 || s->k < 1 || s->I < 1 || s->L < 0 || s->shared_I < 0 ||
      s->capacity < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->dispatch != MOE_DISPATCH_DTYPE && s->dispatch != MOE_DISPATCH_MXFP8) return MOE_ERR_INVALID_ARG;
  if (s->k > s->E) return MOE_ERR_INVALID_ARG;
  if (s->E > kMaxE || s->k > kWave) return MOE_ERR_UNSUPPORTED;
  if (s->T > INT_MAX || s->H > INT_MAX || s->I > INT_MAX || s->L > INT_MAX) return MOE_ERR_UNSUPPORTED;
  if (s->T * s->k > INT_MAX) return MOE_ERR_UNSUPPORTED;
  d.T = (int)s->T; d.H = (int)s->H; d.E = (int)s->E; d.k = (int)s->k; d.I = (int)s->I;
  d.L = (int)s->L; d.D = d.L ? d.L : d.H; d.R = d.T * d.k;
  d.nb = ceil_div(d.T, block_tokens(d.T));
  d.Is = s->shared_I;
  // a token picks an expert at most once, so no expert holds more than T rows
  d.cap = s->capacity >= s->T ? 0 : (int)s->capacity;
  d.bf16 = s->dtype == MOE_BF16;
  d.es = d.bf16 ? 2 : 4;
  d.mx = s->dispatch == MOE_DISPATCH_MXFP8;
  if (d.Is && d.L) return MOE_ERR_UNSUPPORTED;  // shared expert on non-latent layers only
  if (d.mx && (!d.bf16 || d.D % 128)) return MOE_ERR_UNSUPPORTED;  // bf16 layers, 128-code K-steps
  if (d.bf16) {
    if (d.D % 64 || d.I % 64 || (d.L && d.H % 64) || d.Is % 64) return MOE_ERR_UNSUPPORTED;
  } else {
    if (d.D % 4 || d.H % 4 || d.Is % 4) return MOE_ERR_UNSUPPORTED;
  }
  // element counts addressed with int inside some kernels
  if ((long long)d.R * d.D / 8 > INT_MAX || (long long)d.T * d.E > INT_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

GemmKind expert_kind(const Dims& d) {
  if (!d.bf16) return GEMM_SIMT;
  // mean rows per expert decides between one weight pass with 128-row tiles and
  // 16-row tiles that stream weights once per handful of rows
  return (d.R >= 48 * d.E) ? GEMM_PREFILL : GEMM_DECODE;
}

size_t gate_partial_bytes(const Dims& d);

struct RouteWs { size_t bc, gpart, total; };
RouteWs route_ws(const Dims& d, bool with_gate) {
  Carve c; RouteWs w;
  w.bc = c.take((size_t)d.nb * d.E * 4);
  w.gpart = c.take(with_gate ? gate_partial_bytes(d) : 0);
  w.total = c.cur;
  return w;
}

struct FfnWs { size_t mtile, act, total; };
FfnWs ffn_ws(const Dims& d) {
  Carve c; FfnWs w;
  w.mtile = c.take(mtile_table_bytes(d.E));  // tables for two tile heights + claim counters
  w.act = c.take((size_t)d.R * d.I * d.es);
  w.total = c.cur;
  return w;
}

struct CombWs { size_t ytok, total; };
CombWs comb_ws(const Dims& d) {
  Carve c; CombWs w;
  w.ytok = c.take((size_t)d.R * d.D * d.es);
  w.total = c.cur;
  return w;
}

struct LayerWs {
  size_t logits, ids, w, counts, offsets, row_token, token_row, bc, handover, gpart, mtile, z, xperm, act,
      outl, soffs, smtile, sact, sy, xs, xq, xqs, total;
};
LayerWs layer_ws(const Dims& d) {
  Carve c; LayerWs w;
  w.logits = c.take((size_t)d.T * d.E * 4);
  w.ids = c.take((size_t)d.R * 4);
  w.w = c.take((size_t)d.R * 4);
  w.counts = c.take((size_t)d.E * 4);
  w.offsets = c.take((size_t)(d.E + 1) * 4);
  w.row_token = c.take((size_t)d.R * 4);
  w.token_row = c.take((size_t)d.R * 4);
  w.bc = c.take((size_t)d.nb * d.E * 4);
  // decode-scale routing over several workgroups: their hand-over word
  w.handover = c.take(d.T <= kSmallT ? 8 : 0);
  w.gpart = c.take(gate_partial_bytes(d));
  w.mtile = c.take(mtile_table_bytes(d.E));  // tables for two tile heights + claim counters
  w.z = c.take(d.L ? (size_t)d.T * d.L * d.es : 0);
  w.xperm = c.take((size_t)d.R * d.D * d.es);  // later reused for y_perm
  w.xs = c.take(d.mx ? (size_t)d.R * (d.D / kMxBlock) : 0);  // MXFP8 scales of x_perm
  // MXFP8 decode-scale steps: the token rows quantised once, read through row_token
  w.xq = c.take(d.mx ? (size_t)d.T * d.D : 0);
  w.xqs = c.take(d.mx ? (size_t)d.T * (d.D / kMxBlock) : 0);
  w.act = c.take((size_t)d.R * d.I * d.es);
  w.outl = c.take(d.L ? (size_t)d.T * d.L * d.es : 0);
  // shared expert: one group of T rows
  w.soffs = c.take(d.Is ? 2 * 4 : 0);
  w.smtile = c.take(d.Is ? mtile_table_bytes(1) : 0);
  w.sact = c.take((size_t)d.T * d.Is * d.es);
  w.sy = c.take(d.Is ? (size_t)d.T * d.H * d.es : 0);
  w.total = c.cur;
  return w;
}

// The shared expert's FFN as a grouped FFN of one expert over all T rows.
Dims shared_dims(const Dims& d) {
  Dims s = d;
  s.mx = false;  // the shared expert's rows are not dispatched
  s.E = 1;
  s.k = 1;
  s.R = d.T;
  s.I = d.Is;
  s.D = d.H;
  return s;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

#define MOE_HIP(call)                          \
  do {                                         \
    if ((call) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

size_t gate_partial_bytes(const Dims& d) {
  if (!d.bf16) return 0;
  const int s = gate_plan(d.T, d.E, d.H).splits;
  return s > 1 ? (size_t)s * d.T * d.E * 4 : 0;
}

// a1, and where a2 then reads the scores (ScoreSrc): with the gate's output split
// over K the top-k kernel sums the slices and writes the logits itself (one launch
// and one pass over T x E fewer than a separate reduce).
moe_status gate_scores(const Dims& d, const void* x, const float* gate_w, const float* bias,
                       float* logits, float* partial, hipStream_t st, ScoreSrc* src) {
  int S = 1;
  if (d.bf16) {
    MOE_HIP(launch_gate_bf16(static_cast<const uint16_t*>(x), gate_w, bias, logits, partial, d.T, d.E,
                             d.H, st, true, &S));
  } else {
    MOE_HIP(launch_gemm_simt(false, EPI_F32_BIAS, x, d.T, gate_w, nullptr, logits, nullptr, nullptr,
                             1, d.E, d.H, bias, st));
  }
  if (S > 1)
    *src = ScoreSrc{nullptr, partial, S, (size_t)d.T * d.E, bias, logits};
  else  // the gate wrote logits with the bias in them
    *src = ScoreSrc{logits, nullptr, 1, 0, nullptr, nullptr};
  return MOE_OK;
}

// Given router logits: read as they are, the bias (nullable) added on the fly.
ScoreSrc given_scores(const float* logits, const float* bias) {
  return ScoreSrc{logits, nullptr, 1, 0, bias, nullptr};
}

moe_status expert_ffn(const Dims& d, const void* x_perm, const int32_t* offsets,
                      const int32_t* mtile, const void* w1, const void* w3, const void* w2,
                      void* act, void* y_perm, hipStream_t st, MxScales mx = MxScales{}) {
  const GemmKind kind = expert_kind(d);
  if (d.mx) {
    MOE_HIP(launch_gemm_mx_swiglu(kind, static_cast<const uint8_t*>(x_perm), d.R,
                                  static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w3),
                                  static_cast<uint16_t*>(act), offsets, mtile, d.E, d.I, d.D, mx, nullptr,
                                  st));
    MOE_HIP(launch_gemm_bf16(kind, EPI_BF16, static_cast<const uint16_t*>(act), d.R,
                             static_cast<const uint16_t*>(w2), nullptr, y_perm, offsets, mtile,
                             d.E, d.D, d.I, st));
  } else if (kind == GEMM_SIMT) {
    MOE_HIP(launch_gemm_simt(false, EPI_SWIGLU_F32, x_perm, d.R, static_cast<const float*>(w1),
                             static_cast<const float*>(w3), act, offsets, mtile, d.E, d.I, d.D,
                             nullptr, st));
    MOE_HIP(launch_gemm_simt(false, EPI_F32, act, d.R, static_cast<const float*>(w2), nullptr,
                             y_perm, offsets, mtile, d.E, d.D, d.I, nullptr, st));
  } else {
    MOE_HIP(launch_gemm_bf16(kind, EPI_SWIGLU_BF16, static_cast<const uint16_t*>(x_perm), d.R,
                             static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3),
                             act, offsets, mtile, d.E, d.I, d.D, st));
    MOE_HIP(launch_gemm_bf16(kind, EPI_BF16, static_cast<const uint16_t*>(act), d.R,
                             static_cast<const uint16_t*>(w2), nullptr, y_perm, offsets, mtile,
                             d.E, d.D, d.I, st));
  }
  return MOE_OK;
}

// Dense projection C[M x N] = A[M x K] W^T for the latent layers (W stored [N x K]).
moe_status dense_proj(const Dims& d, const void* A, const void* W, void* C, int M, int N, int K,
                      bool out_f32, hipStream_t st) {
  if (d.bf16) {
    MOE_HIP(launch_gemm_bf16(GEMM_PREFILL, out_f32 ? EPI_F32 : EPI_BF16,
                             static_cast<const uint16_t*>(A), M, static_cast<const uint16_t*>(W),
                             nullptr, C, nullptr, nullptr, 1, N, K, st));
  } else {
    if (!out_f32) return MOE_ERR_UNSUPPORTED;
    MOE_HIP(launch_gemm_simt(false, EPI_F32, A, M, static_cast<const float*>(W), nullptr, C,
                             nullptr, nullptr, 1, N, K, nullptr, st));
  }
  return MOE_OK;
}

// Tags of the decode-scale router's hand-over word: distinct for every call in the
// process, never 0 (the router clears the word to 0 after use), below 2^56.
std::atomic<unsigned long long> g_route_tag{1};
unsigned long long next_route_tag() {
  return (g_route_tag.fetch_add(1, std::memory_order_relaxed) - 1) % ((1ull << 56) - 1) + 1;
}

// Every decision moe_layer_forward takes from the shape and from which optional buffers
// the caller passes; moe_layer_plan reports the same struct.
struct LayerPlan {
  GemmKind kind;
  bool small;  // decode-scale routing in one launch, gate/up reading the token rows
  bool gath;   // larger steps: the permutation writes metadata only, gate/up gathers the rows
  bool fused_dc;  // decode-scale steps: the down GEMM and the combine in one launch
  GemmChoice gate_up, down, shared_gate_up, shared_down;
  int launches;
};

LayerPlan plan_layer(const Dims& d, bool gate_computed, bool want_xperm, bool want_xperm_scale) {
  LayerPlan p{};
  p.kind = expert_kind(d);
  // Decode-scale steps (16-row expert tiles, T <= kSmallT): routing, counts, offsets,
  // tile tables and row metadata in one launch, and the gate/up GEMM reads its rows
  // straight from the token rows through row_token (no permuted copy unless the
  // caller asks for it in aux.x_perm).  With MXFP8 dispatch the token rows are
  // quantised once and read the same way; a caller who asks for the permuted codes
  // gets the general path.
  // The routing runs in one workgroup while its ranking work is small, each wave ranking
  // ceil(T / 16) tokens one after another (route_one_workgroup); above that, over
  // ceil(T / 4) workgroups, one token per wave, the last to finish writing the metadata.
  p.small = p.kind == GEMM_DECODE && d.T <= kSmallT && !(d.mx && (want_xperm || want_xperm_scale));
  // Larger steps: unless the caller asks for the permuted rows, the permutation writes
  // only the row metadata and the gate/up GEMM reads the token rows through row_token
  // (decode-sized tiles always can; the persistent prefill kernel when its tile table
  // fits).  The GEMM sees the same rows in the same order, so the results are the same
  // bits as with the permuted copy.
  p.gath = !p.small && d.bf16 && !want_xperm && !(d.mx && want_xperm_scale) &&
           (p.kind == GEMM_DECODE ||
            (p.kind == GEMM_PREFILL && gemm_gather_ok(d.R, d.E, d.I, d.mx ? d.D / 2 : d.D, d.mx)));
  p.gate_up = choose_gemm(p.kind, true, true, d.mx, d.R, d.E, d.I, d.mx ? d.D / 2 : d.D);
  p.down = choose_gemm(p.kind, false, true, false, d.R, d.E, d.D, d.I);
  // Decode-scale steps: each workgroup runs the down GEMM for a 16-column slice of every
  // row and combines those columns itself, so the combine needs no launch of its own
  // (and no data passes between workgroups).  Not with a shared expert, whose term the
  // combine adds after the routed ones.
  p.fused_dc = p.kind == GEMM_DECODE && d.bf16 && !d.Is && down_combine_ok(d.R, d.E, d.D, d.I);
  if (p.fused_dc) p.down = GemmChoice{GV_DOWN_COMBINE, 16, 16, false, "k_down_combine<16,"};
  int n = 0;
  if (d.L) n += 1;                            // latent down-projection
  if (gate_computed) n += 1;                  // gate scores (split-K slices summed by the top-k kernel)
  if (p.small) {
    n += 1;                                   // routing, counts, offsets, tile tables, row metadata
    if (d.mx || want_xperm) n += 1;           // token rows quantised once / permuted copy on request
  } else {
    n += 3;                                   // top-k + counts, expert scan, permutation
    if (p.gath && d.mx) n += 1;               // token rows quantised once
  }
  n += 2;                                     // expert gate/up and down GEMMs
  if (d.Is) {
    const Dims ds = shared_dims(d);
    p.shared_gate_up = choose_gemm(expert_kind(ds), true, true, false, ds.R, 1, ds.I, ds.D);
    p.shared_down = choose_gemm(expert_kind(ds), false, true, false, ds.R, 1, ds.D, ds.I);
    n += 3;                                   // its one-group table and two GEMMs
  }
  if (!p.fused_dc) n += 1;                    // combine (inside the down GEMM's launch when fused)
  if (d.L) n += 1;                            // latent up-projection
  p.launches = n;
  return p;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: bad shape or pointer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the kernels' limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe_status";
  }
}

size_t moe_workspace_bytes(const moe_shape* s, int call) {
  Dims d;
  if (check_shape(s, d) != MOE_OK) return 0;
  switch (call) {
    case MOE_CALL_ROUTE: return route_ws(d, true).total;
    case MOE_CALL_DISPATCH: return route_ws(d, false).total;
    case MOE_CALL_FFN: return ffn_ws(d).total;
    case MOE_CALL_COMBINE: return comb_ws(d).total;
    case MOE_CALL_LAYER: return layer_ws(d).total;
    default: return 0;
  }
}

moe_status moe_layer_plan(const moe_shape* s, int flags, moe_plan* out) {
  Dims d;
  moe_status rc = check_shape(s, d);
  if (rc != MOE_OK) return rc;
  if (!out || (flags & ~(MOE_PLAN_GATE | MOE_PLAN_X_PERM))) return MOE_ERR_INVALID_ARG;
  const bool xp = (flags & MOE_PLAN_X_PERM) != 0;
  const LayerPlan p = plan_layer(d, (flags & MOE_PLAN_GATE) != 0, xp, xp && d.mx);
  *out = moe_plan{};
  out->launches = p.launches;
  out->decode_path = p.small;
  out->rows_gathered = p.small || p.gath;
  out->gate_up_tile_m = p.gate_up.bm;
  out->gate_up_tile_n = p.gate_up.bn;
  out->gate_up_persistent = p.gate_up.persistent;
  out->down_tile_m = p.down.bm;
  out->down_tile_n = p.down.bn;
  out->down_persistent = p.down.persistent;
  out->route_workgroups = !p.small ? 0 : route_one_workgroup(d.T, d.E, d.k) ? 1 : ceil_div(d.T, kMultiTok);
  out->gate_up_kernel = p.gate_up.kernel;
  out->down_kernel = p.down.kernel;
  return MOE_OK;
}

moe_status moe_route_topk(const void* x, const float* gate_w, const float* gate_bias,
                          float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                          int32_t* offsets, const moe_shape* s, void* ws, size_t ws_bytes,
                          void* stream) {
  Dims d;
  moe_status rc = check_shape(s, d);
  if (rc != MOE_OK) return rc;
  if (!al16(logits) || !al16(topk_ids) || !al16(topk_w) || !al16(counts) || !al16(offsets) ||
      !al16_or_null(gate_w) || !al16_or_null(gate_bias))
    return MOE_ERR_INVALID_ARG;
  if (gate_w && !al16(x)) return MOE_ERR_INVALID_ARG;
  const RouteWs w = route_ws(d, gate_w != nullptr);
  if (!ws || ws_bytes < w.total || !al16(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ScoreSrc src = given_scores(logits, gate_bias);
  if (gate_w) {
    rc = gate_scores(d, x, gate_w, gate_bias, logits, at<float>(ws, w.gpart), st, &src);
    if (rc != MOE_OK) return rc;
  }
  int32_t* bc = at<int32_t>(ws, w.bc);
  MOE_HIP(launch_topk(src, d.T, d.E, d.k, topk_ids, topk_w, bc, st));
  MOE_HIP(launch_expert_scan(bc, d.nb, d.E, d.cap, counts, st));
  MOE_HIP(launch_offsets(counts, nullptr, d.E, offsets, 0, nullptr, st));
  return MOE_OK;
}

moe_status moe_dispatch_permute(const void* x, const int32_t* topk_ids, const int32_t* offsets,
                                void* x_perm, uint8_t* x_perm_scale, int32_t* row_token, int32_t* token_row,
                                const moe_shape* s, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status rc = check_shape(s, d);
  if (rc != MOE_OK) return rc;
  if (!al16(x) || !al16(topk_ids) || !al16(offsets) || !al16(x_perm) || !al16(row_token) ||
      !al16(token_row) || (d.mx ? !al16(x_perm_scale) : x_perm_scale != nullptr))
    return MOE_ERR_INVALID_ARG;
  const RouteWs w = route_ws(d, false);
  if (!ws || ws_bytes < w.total || !al16(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* bc = at<int32_t>(ws, w.bc);
  MOE_HIP(launch_block_counts(topk_ids, d.T, d.E, d.k, bc, st));
  MOE_HIP(launch_expert_scan(bc, d.nb, d.E, d.cap, nullptr, st));
  MOE_HIP(launch_permute(x, d.D * d.es / 16, topk_ids, d.T, d.E, d.k, d.cap, offsets, bc, x_perm,
                         d.mx ? x_perm_scale : nullptr, row_token, token_row, st));
  return MOE_OK;
}

moe_status moe_grouped_ffn(const void* x_perm, const uint8_t* x_perm_scale, const int32_t* offsets,
                           const void* w1, const uint8_t* w1_scale, const void* w3, const uint8_t* w3_scale,
                           const void* w2, void* y_perm, const moe_shape* s, void* ws, size_t ws_bytes,
                           void* stream) {
  Dims d;
  moe_status rc = check_shape(s, d);
  if (rc != MOE_OK) return rc;
  if (!al16(x_perm) || !al16(offsets) || !al16(w1) || !al16(w3) || !al16(w2) || !al16(y_perm))
    return MOE_ERR_INVALID_ARG;
  if (d.mx ? (!al16(x_perm_scale) || !al16(w1_scale) || !al16(w3_scale))
           : (x_perm_scale || w1_scale || w3_scale))
    return MOE_ERR_INVALID_ARG;
  const FfnWs w = ffn_ws(d);
  if (!ws || ws_bytes < w.total || !al16(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* mtile = at<int32_t>(ws, w.mtile);
  MOE_HIP(launch_offsets(nullptr, offsets, d.E, nullptr, gemm_bm(expert_kind(d)), mtile, st));
  return expert_ffn(d, x_perm, offsets, mtile, w1, w3, w2, at<void>(ws, w.act), y_perm, st,
                    MxScales{x_perm_scale, w1_scale, w3_scale});
}

moe_status moe_quantize_mxfp8(const void* src, int src_dtype, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* scale, void* stream) {
  if (rows < 0 || cols < 1 || (src_dtype != MOE_F32 && src_dtype != MOE_BF16)) return MOE_ERR_INVALID_ARG;
  if (cols % kMxBlock) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!al16(src) || !al16(q) || !al16(scale)) return MOE_ERR_INVALID_ARG;
  if (rows > (int64_t)1 << 40 || cols > INT_MAX) return MOE_ERR_UNSUPPORTED;
  MOE_HIP(launch_mx_quantize(src, src_dtype == MOE_BF16, (long)rows, (long)cols, q, scale,
                             static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_combine(const void* y_perm, const int32_t* token_row, const float* topk_w,
                       const void* shared_out, void* out, int out_dtype, int flags,
                       const moe_shape* s, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status rc = check_shape(s, d);
  if (rc != MOE_OK) return rc;
  if (!al16(y_perm) || !al16(token_row) || !al16(topk_w) || !al16(out) || !al16_or_null(shared_out))
    return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (flags != MOE_COMBINE_FUSED && flags != MOE_COMBINE_UNFUSED) return MOE_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int row16 = d.D * d.es / 16;
  const bool of32 = out_dtype == MOE_F32;
  if (flags == MOE_COMBINE_FUSED) {
    MOE_HIP(launch_combine(y_perm, row16, d.bf16, token_row, topk_w, shared_out, d.T, d.k, out, of32,
                           st));
    return MOE_OK;
  }
  const CombWs w = comb_ws(d);
  if (!ws || ws_bytes < w.total || !al16(ws)) return MOE_ERR_WORKSPACE;
  void* ytok = at<void>(ws, w.ytok);
  MOE_HIP(launch_unpermute(y_perm, row16, token_row, d.R, nullptr, ytok, st));
  MOE_HIP(launch_weighted_reduce(ytok, row16, d.bf16, token_row, topk_w, shared_out, d.T, d.k, out,
                                 of32, st));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_layer_weights* wt, const void* x, float* logits, void* out,
                             int out_dtype, const moe_shape* s, moe_layer_aux* aux,
                             void** stage_events, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status rc = check_shape(s, d);
  if (rc != MOE_OK) return rc;
  if (!wt || !al16(x) || !al16(out) || !al16(wt->w1) || !al16(wt->w3) || !al16(wt->w2))
    return MOE_ERR_INVALID_ARG;
  if (!al16_or_null(wt->gate_w) || !al16_or_null(wt->gate_bias) || !al16_or_null(logits))
    return MOE_ERR_INVALID_ARG;
  if (!wt->gate_w && !logits) return MOE_ERR_INVALID_ARG;  // given logits are required
  if (d.L && (!al16(wt->wd) || !al16(wt->wu))) return MOE_ERR_INVALID_ARG;
  if (d.Is && (!al16(wt->ws1) || !al16(wt->ws3) || !al16(wt->ws2))) return MOE_ERR_INVALID_ARG;
  if (d.mx ? (!al16(wt->w1_scale) || !al16(wt->w3_scale)) : (wt->w1_scale || wt->w3_scale))
    return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!d.bf16 && d.L && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  moe_layer_aux none = {};
  moe_layer_aux& ax = aux ? *aux : none;
  if (!d.mx && ax.x_perm_scale) return MOE_ERR_INVALID_ARG;
  const void* auxp[] = {ax.topk_ids, ax.topk_w, ax.counts, ax.offsets, ax.row_token,
                        ax.token_row, ax.x_perm, ax.y_perm, ax.z, ax.out_latent, ax.x_perm_scale};
  for (const void* p : auxp)
    if (!al16_or_null(p)) return MOE_ERR_INVALID_ARG;
  const LayerWs w = layer_ws(d);
  if (!ws || ws_bytes < w.total || !al16(ws)) return MOE_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  auto pick = [&](void* user, size_t off) { return user ? user : at<void>(ws, off); };
  float* lg = static_cast<float*>(logits ? logits : at<void>(ws, w.logits));
  int32_t* ids = static_cast<int32_t*>(pick(ax.topk_ids, w.ids));
  float* tw = static_cast<float*>(pick(ax.topk_w, w.w));
  int32_t* counts = static_cast<int32_t*>(pick(ax.counts, w.counts));
  int32_t* offs = static_cast<int32_t*>(pick(ax.offsets, w.offsets));
  int32_t* rtok = static_cast<int32_t*>(pick(ax.row_token, w.row_token));
  int32_t* trow = static_cast<int32_t*>(pick(ax.token_row, w.token_row));
  int32_t* bc = at<int32_t>(ws, w.bc);
  int32_t* mtile = at<int32_t>(ws, w.mtile);
  void* z = d.L ? pick(ax.z, w.z) : nullptr;
  void* xperm = pick(ax.x_perm, w.xperm);
  // y_perm: caller's buffer, else the workspace x_perm region (free once the gate/up GEMM has read it)
  void* yperm = ax.y_perm ? ax.y_perm : at<void>(ws, w.xperm);
  void* act = at<void>(ws, w.act);
  void* outl = d.L ? pick(ax.out_latent, w.outl) : nullptr;
  uint8_t* xs = d.mx ? static_cast<uint8_t*>(pick(ax.x_perm_scale, w.xs)) : nullptr;

  auto ev = [&](int i) -> bool {
    return !stage_events || !stage_events[i] ||
           hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), st) == hipSuccess;
  };
  const LayerPlan plan = plan_layer(d, wt->gate_w != nullptr, ax.x_perm != nullptr, ax.x_perm_scale != nullptr);
  const GemmKind kind = plan.kind;

  if (!ev(0)) return MOE_ERR_HIP;
  if (d.L) {  // a7: Z = X wd^T (rounded to the layer dtype)
    rc = dense_proj(d, x, wt->wd, z, d.T, d.L, d.H, !d.bf16, st);
    if (rc != MOE_OK) return rc;
  }
  if (!ev(1)) return MOE_ERR_HIP;
  ScoreSrc scores = given_scores(lg, wt->gate_bias);
  if (wt->gate_w) {  // a1: router logits on the full-width state
    rc = gate_scores(d, x, wt->gate_w, wt->gate_bias, lg, at<float>(ws, w.gpart), st, &scores);
    if (rc != MOE_OK) return rc;
  }
  if (!ev(2)) return MOE_ERR_HIP;
  const void* src = d.L ? z : x;  // the rows that are dispatched
  const int row16 = d.D * d.es / 16;
  const bool small = plan.small, gath = plan.gath;
  const bool rows_from_tokens = small || gath;
  // a5 down GEMM (bf16), or on decode-scale steps the down GEMM with the combine (a6)
  auto down_bf16 = [&]() -> hipError_t {
    if (plan.fused_dc)
      return launch_down_combine(static_cast<const uint16_t*>(act), d.R, static_cast<const uint16_t*>(wt->w2),
                                 offs, mtile, d.E, d.D, d.I, trow, tw, nullptr, d.T, d.k, d.L ? outl : out,
                                 d.L ? !d.bf16 : out_dtype == MOE_F32, ax.y_perm, st);
    return launch_gemm_bf16(kind, EPI_BF16, static_cast<const uint16_t*>(act), d.R,
                            static_cast<const uint16_t*>(wt->w2), nullptr, yperm, offs, mtile, d.E, d.D, d.I,
                            st);
  };
  uint8_t* xq = d.mx ? at<uint8_t>(ws, w.xq) : nullptr;
  uint8_t* xqs = d.mx ? at<uint8_t>(ws, w.xqs) : nullptr;
  if (small) {
    MOE_HIP(launch_route_small(scores, d.T, d.E, d.k, ids, tw, counts, offs, rtok, trow, d.cap,
                               gemm_bm(kind), mtile, at<unsigned long long>(ws, w.handover),
                               next_route_tag(), st));
    if (!ev(3)) return MOE_ERR_HIP;
    if (d.mx) {
      MOE_HIP(launch_mx_quantize(src, true, d.T, d.D, xq, xqs, st));
    } else if (ax.x_perm) {  // rows [0, offsets[E]) are the kept ones
      MOE_HIP(launch_unpermute(src, row16, rtok, d.R, offs + d.E, ax.x_perm, st));
    }
  } else {
    // a2 + a3
    MOE_HIP(launch_topk(scores, d.T, d.E, d.k, ids, tw, bc, st));
    MOE_HIP(launch_expert_scan(bc, d.nb, d.E, d.cap, counts, st));
    if (!ev(3)) return MOE_ERR_HIP;
    // a3 (segment starts, GEMM tile tables) inside the a4 launch
    const PermuteOffsets po{counts, offs, gemm_bm(kind), mtile};
    if (gath) {
      if (d.mx) MOE_HIP(launch_mx_quantize(src, true, d.T, d.D, xq, xqs, st));  // token rows, once
      MOE_HIP(launch_permute(src, row16, ids, d.T, d.E, d.k, d.cap, offs, bc, nullptr, nullptr, rtok, trow, st, &po));
    } else {
      MOE_HIP(launch_permute(src, row16, ids, d.T, d.E, d.k, d.cap, offs, bc, xperm, xs, rtok, trow, st, &po));
    }
  }
  if (!ev(4)) return MOE_ERR_HIP;
  // a5
  if (d.mx) {
    const MxScales mx{rows_from_tokens ? xqs : xs, wt->w1_scale, wt->w3_scale};
    MOE_HIP(launch_gemm_mx_swiglu(kind, static_cast<const uint8_t*>(rows_from_tokens ? xq : xperm), d.R,
                                  static_cast<const uint8_t*>(wt->w1), static_cast<const uint8_t*>(wt->w3),
                                  static_cast<uint16_t*>(act), offs, mtile, d.E, d.I, d.D, mx,
                                  rows_from_tokens ? rtok : nullptr, st));
    if (!ev(5)) return MOE_ERR_HIP;
    MOE_HIP(down_bf16());
  } else if (rows_from_tokens) {
    if (kind == GEMM_DECODE)
      MOE_HIP(launch_gemm_decode_gather(EPI_SWIGLU_BF16, static_cast<const uint16_t*>(src), rtok, d.R,
                                        static_cast<const uint16_t*>(wt->w1),
                                        static_cast<const uint16_t*>(wt->w3), act, offs, mtile, d.E, d.I,
                                        d.D, st));
    else
      MOE_HIP(launch_gemm_prefill_gather(EPI_SWIGLU_BF16, static_cast<const uint16_t*>(src), rtok, d.R,
                                         static_cast<const uint16_t*>(wt->w1),
                                         static_cast<const uint16_t*>(wt->w3), act, offs, mtile, d.E, d.I,
                                         d.D, st));
    if (!ev(5)) return MOE_ERR_HIP;
    MOE_HIP(down_bf16());
  } else if (kind == GEMM_SIMT) {
    MOE_HIP(launch_gemm_simt(false, EPI_SWIGLU_F32, xperm, d.R, static_cast<const float*>(wt->w1),
                             static_cast<const float*>(wt->w3), act, offs, mtile, d.E, d.I, d.D,
                             nullptr, st));
    if (!ev(5)) return MOE_ERR_HIP;
    MOE_HIP(launch_gemm_simt(false, EPI_F32, act, d.R, static_cast<const float*>(wt->w2), nullptr,
                             yperm, offs, mtile, d.E, d.D, d.I, nullptr, st));
  } else {
    MOE_HIP(launch_gemm_bf16(kind, EPI_SWIGLU_BF16, static_cast<const uint16_t*>(xperm), d.R,
                             static_cast<const uint16_t*>(wt->w1),
                             static_cast<const uint16_t*>(wt->w3), act, offs, mtile, d.E, d.I, d.D,
                             st));
    if (!ev(5)) return MOE_ERR_HIP;
    MOE_HIP(down_bf16());
  }
  if (!ev(6)) return MOE_ERR_HIP;
  // shared expert: every token, whatever the router picked
  void* sy = nullptr;
  if (d.Is) {
    const Dims ds = shared_dims(d);
    int32_t* soffs = at<int32_t>(ws, w.soffs);
    int32_t* smtile = at<int32_t>(ws, w.smtile);
    sy = at<void>(ws, w.sy);
    MOE_HIP(launch_single_group(d.T, soffs, gemm_bm(expert_kind(ds)), smtile, st));
    rc = expert_ffn(ds, x, soffs, smtile, wt->ws1, wt->ws3, wt->ws2, at<void>(ws, w.sact), sy, st);
    if (rc != MOE_OK) return rc;
  }
  if (!ev(7)) return MOE_ERR_HIP;
  // a6 (on fused decode-scale steps it ran inside the down GEMM's launch)
  if (!plan.fused_dc) {
    if (d.L)
      MOE_HIP(launch_combine(yperm, row16, d.bf16, trow, tw, nullptr, d.T, d.k, outl, !d.bf16, st));
    else
      MOE_HIP(launch_combine(yperm, row16, d.bf16, trow, tw, sy, d.T, d.k, out, out_dtype == MOE_F32, st));
  }
  if (!ev(8)) return MOE_ERR_HIP;
  if (d.L) {  // a7: out = out_L wu^T
    rc = dense_proj(d, outl, wt->wu, out, d.T, d.H, d.L, out_dtype == MOE_F32, st);
    if (rc != MOE_OK) return rc;
  }
  if (!ev(9)) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // extern "C"
