/* Host-side exercise of the libmoe C ABI for an AddressSanitizer build (no GPU work).
 *
 * Every call below either is host-only (moe_workspace_bytes, moe_layer_plan,
 * moe_status_string, moe_abi_version) or fails its host-side argument validation, so
 * it returns before any HIP call; the fake device pointers are never dereferenced.
 * Exit status 0 when every status is the documented one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond);   \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static moe_shape shape(int64_t T, int64_t H, int64_t E, int64_t k, int64_t I, int64_t L, int bf16) {
  moe_shape s;
  memset(&s, 0, sizeof s);
  s.T = T; s.H = H; s.E = E; s.k = k; s.I = I; s.L = L;
  s.dtype = bf16 ? MOE_BF16 : MOE_F32;
  return s;
}

int main(void) {
  void* F = (void*)(uintptr_t)0x10000; /* aligned, never dereferenced */
  EXPECT(moe_abi_version() == MOE_ABI_VERSION);
  for (int c = -1; c < 7; ++c) EXPECT(moe_status_string(c) != NULL && strlen(moe_status_string(c)) > 0);

  /* workspace sizes and plans over a spread of shapes, including the full-size layers */
  const int64_t shapes[][7] = {
      {64, 128, 8, 2, 256, 0, 0},        {4096, 2048, 128, 8, 768, 0, 1}, {8192, 7168, 256, 8, 2048, 0, 1},
      {128, 4096, 896, 16, 1024, 0, 1},  {4096, 7168, 256, 8, 4096, 2048, 1}, {1, 64, 1, 1, 64, 0, 1},
      {131072, 64, 1024, 64, 64, 0, 1},  {524289, 256, 1, 1, 128, 0, 1},  {8, 4096, 896, 16, 1024, 0, 1}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    moe_shape s = shape(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4], shapes[i][5],
                        (int)shapes[i][6]);
    for (int call = 0; call <= MOE_CALL_LAYER; ++call) EXPECT(moe_workspace_bytes(&s, call) > 0);
    EXPECT(moe_workspace_bytes(&s, 99) == 0);
    for (int flags = 0; flags < 4; ++flags) {
      moe_plan p;
      memset(&p, 0xff, sizeof p);
      EXPECT(moe_layer_plan(&s, flags, &p) == MOE_OK);
      EXPECT(p.launches >= 3 && p.gate_up_kernel && p.down_kernel && strlen(p.gate_up_kernel) > 0);
    }
    moe_plan p;
    EXPECT(moe_layer_plan(&s, 4, &p) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_layer_plan(&s, 0, NULL) == MOE_ERR_INVALID_ARG);
  }
  moe_shape bad = shape(0, 128, 8, 2, 256, 0, 1);
  EXPECT(moe_workspace_bytes(&bad, MOE_CALL_LAYER) == 0);
  EXPECT(moe_workspace_bytes(NULL, MOE_CALL_LAYER) == 0);
  moe_plan p;
  EXPECT(moe_layer_plan(&bad, 0, &p) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_plan(NULL, 0, &p) == MOE_ERR_INVALID_ARG);

  /* every compute call rejects bad arguments on the host */
  moe_shape s = shape(64, 128, 8, 2, 256, 0, 1);
  EXPECT(moe_route_topk(F, NULL, NULL, NULL, F, F, F, F, &s, F, 1 << 20, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(F, NULL, NULL, F, F, F, F, F, &s, F, 16, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_route_topk(F, NULL, NULL, F, F, F, F, F, &bad, F, 1 << 20, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(F, NULL, NULL, F, (void*)((char*)F + 4), F, F, F, &s, F, 1 << 20, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_dispatch_permute(F, F, F, NULL, NULL, F, F, &s, F, 1 << 20, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_dispatch_permute(F, F, F, F, NULL, F, F, &s, F, 0, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_grouped_ffn(F, NULL, F, F, NULL, F, NULL, NULL, F, &s, F, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_ffn(F, NULL, F, F, NULL, F, NULL, F, F, &s, F, 8, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_combine(F, F, F, NULL, F, 5, 0, &s, F, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(F, F, F, NULL, F, 0, 3, &s, F, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(F, F, F, NULL, F, 0, MOE_COMBINE_UNFUSED, &s, F, 8, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_quantize_mxfp8(F, MOE_BF16, 4, 48, F, F, NULL) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_quantize_mxfp8(NULL, MOE_BF16, 0, 64, NULL, NULL, NULL) == MOE_OK);
  moe_layer_weights w;
  memset(&w, 0, sizeof w);
  w.w1 = F; w.w3 = F; w.w2 = F;
  moe_layer_aux aux;
  memset(&aux, 0, sizeof aux);
  EXPECT(moe_layer_forward(&w, F, NULL, F, MOE_F32, &s, &aux, NULL, F, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward(&w, F, F, F, MOE_F32, &s, &aux, NULL, F, 1024, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_forward(NULL, F, F, F, MOE_F32, &s, &aux, NULL, F, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  aux.x_perm = (void*)((char*)F + 8);
  EXPECT(moe_layer_forward(&w, F, F, F, MOE_F32, &s, &aux, NULL, F, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);

  /* the allocation-free variant: validation, then the scratch-size limit, on the host */
  aux.x_perm = NULL;
  EXPECT(moe_layer_forward_noalloc(&w, F, NULL, F, MOE_F32, &s, &aux, NULL, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward_noalloc(&w, F, F, F, MOE_F32, &bad, &aux, NULL, NULL) == MOE_ERR_INVALID_ARG);
  moe_shape huge = shape(8192, 7168, 256, 8, 2048, 0, 1);
  EXPECT(moe_workspace_bytes(&huge, MOE_CALL_LAYER) > MOE_NOALLOC_SCRATCH_BYTES);
  EXPECT(moe_layer_forward_noalloc(&w, F, F, F, MOE_F32, &huge, &aux, NULL, NULL) == MOE_ERR_WORKSPACE);

  if (failures) fprintf(stderr, "%d failure(s)\n", failures);
  else printf("abi host driver: all checks passed\n");
  return failures ? 1 : 0;
}
