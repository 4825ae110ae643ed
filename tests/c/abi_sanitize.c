/*
 * The library's host code (argument checks, workspace planning, metadata and
 * profiling bookkeeping) under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every call here is answered on the host before any GPU work, so it runs on a
 * machine without a GPU.  It sweeps the workspace planner over shapes up to the
 * ABI's limits (sizes must be positive, 256-byte multiples and grow with the
 * token count), and drives every entry point through its argument errors.
 * Prints one line per check and exits nonzero on a failed check; a sanitizer
 * report aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kt_rawint4.h"

#define FAKE ((const void*)(uintptr_t)(1u << 20)) /* 256-byte aligned, never dereferenced */
#define ODD ((const void*)(uintptr_t)((1u << 20) + 2))

static int fails = 0, checks = 0;
static void check(int ok, const char* what) {
  ++checks;
  if (!ok) {
    printf("FAIL %s (%s)\n", what, kt_rawint4_last_error());
    ++fails;
  }
}

static kt_rawint4_moe_layer layer(int E, int k, int H, int I, int r) {
  kt_rawint4_moe_layer L;
  memset(&L, 0, sizeof L);
  L.num_experts = E;
  L.top_k = k;
  L.hidden = H;
  L.intermediate = I;
  L.rank = r;
  L.alpha = 2.f * (float)r;
  L.swiglu_limit = 7.f;
  L.gate_packed = L.up_packed = L.down_packed = (const uint8_t*)FAKE;
  L.gate_scale = L.up_scale = L.down_scale = (const uint16_t*)FAKE;
  L.gate_lora_a = L.gate_lora_b = L.up_lora_a = L.up_lora_b = L.down_lora_a = L.down_lora_b = (const float*)FAKE;
  return L;
}

static void base_only(kt_rawint4_moe_layer* L) {
  L->gate_lora_a = L->gate_lora_b = L->up_lora_a = L->up_lora_b = L->down_lora_a = L->down_lora_b = NULL;
}

static void sweep_planner(void) {
  const int Es[] = {1, 4, 384, 8192};
  const int ks[] = {1, 2, 8};
  const int dims[][2] = {{32, 32}, {96, 160}, {7168, 2048}, {65536, 32}};
  const int ranks[] = {1, 5, 16, 64, 128};
  const int qlens[] = {0, 1, 5, 4096, 16384};
  int n = 0;
  for (size_t a = 0; a < sizeof Es / sizeof *Es; ++a)
    for (size_t b = 0; b < sizeof ks / sizeof *ks; ++b)
      for (size_t c = 0; c < sizeof dims / sizeof *dims; ++c)
        for (size_t d = 0; d < sizeof ranks / sizeof *ranks; ++d) {
          if (ks[b] > Es[a]) continue;
          kt_rawint4_moe_layer L = layer(Es[a], ks[b], dims[c][0], dims[c][1], ranks[d]);
          size_t prev_train = 0, prev_inf = 0;
          for (size_t q = 0; q < sizeof qlens / sizeof *qlens; ++q) {
            const size_t tr = kt_rawint4_moe_workspace_bytes(&L, qlens[q]);
            const size_t inf = kt_rawint4_moe_infer_workspace_bytes(&L, qlens[q]);
            check(tr > 0 && tr % 256 == 0 && tr >= prev_train, "training workspace size");
            check(inf > 0 && inf % 256 == 0 && inf <= tr && inf >= prev_inf, "inference workspace size");
            kt_rawint4_moe_layer B = L;
            base_only(&B);
            check(kt_rawint4_moe_infer_workspace_bytes(&B, qlens[q]) <= inf, "base-only workspace size");
            L.weight_format = KT_RAWINT4_FORMAT_MXFP4;
            check(kt_rawint4_moe_workspace_bytes(&L, qlens[q]) == tr, "MXFP4 workspace size");
            L.weight_format = KT_RAWINT4_FORMAT_RAWINT4;
            check(kt_rawint4_group_workspace_bytes(qlens[q], ks[b], Es[a]) > 0, "grouping workspace size");
            prev_train = tr;
            prev_inf = inf;
            ++n;
          }
        }
  printf("ok   workspace planner over %d shapes\n", n);
}

static void argument_errors(void) {
  const kt_rawint4_moe_layer good = layer(8, 2, 512, 384, 8);
  kt_rawint4_moe_layer L;
  float* g = (float*)FAKE;
  uint16_t* o = (uint16_t*)FAKE;
  const size_t need = kt_rawint4_moe_workspace_bytes(&good, 4);

#define BAD_LAYER(field, value, what)                                                                        \
  do {                                                                                                       \
    L = good;                                                                                                \
    L.field = value;                                                                                         \
    check(kt_rawint4_moe_workspace_bytes(&L, 4) == 0, what " (size)");                                       \
    check(kt_rawint4_moe_fwd(&L, 4, FAKE, FAKE, FAKE, o, (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,       \
          what " (fwd)");                                                                                    \
    check(kt_rawint4_moe_infer_static(&L, 4, FAKE, FAKE, FAKE, o, NULL) == KT_RAWINT4_EINVAL,                \
          what " (static)");                                                                                 \
    check(kt_rawint4_moe_bwd(&L, 4, FAKE, FAKE, FAKE, FAKE, o, NULL, g, g, g, g, g, g, 0, 1.f, (void*)FAKE,  \
                             need, NULL) == KT_RAWINT4_EINVAL,                                               \
          what " (bwd)");                                                                                    \
  } while (0)

  BAD_LAYER(num_experts, 0, "no experts");
  BAD_LAYER(num_experts, KT_RAWINT4_MAX_EXPERTS + 1, "too many experts");
  BAD_LAYER(top_k, 9, "top_k above the experts");
  BAD_LAYER(top_k, 0, "top_k zero");
  BAD_LAYER(hidden, 500, "hidden not a multiple of 32");
  BAD_LAYER(hidden, 65536 + 32, "hidden too large");
  BAD_LAYER(intermediate, -32, "negative intermediate");
  BAD_LAYER(rank, 0, "rank zero");
  BAD_LAYER(rank, KT_RAWINT4_MAX_RANK + 1, "rank too large");
  BAD_LAYER(alpha, NAN, "alpha NaN");
  BAD_LAYER(swiglu_limit, -1.f, "negative limit");
  BAD_LAYER(swiglu_limit, INFINITY, "infinite limit");
  BAD_LAYER(weight_format, 2, "unknown weight format");
  BAD_LAYER(gate_packed, NULL, "missing weights");
  BAD_LAYER(down_scale, NULL, "missing scales");
  BAD_LAYER(up_lora_b, NULL, "one missing LoRA tensor");
  BAD_LAYER(up_packed, (const uint8_t*)ODD, "misaligned weights");
  BAD_LAYER(gate_lora_a, (const float*)ODD, "misaligned LoRA tensor");

  check(kt_rawint4_moe_workspace_bytes(NULL, 4) == 0, "NULL layer (size)");
  check(kt_rawint4_moe_fwd(NULL, 4, FAKE, FAKE, FAKE, o, (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,
        "NULL layer (fwd)");
  check(kt_rawint4_moe_fwd(&good, -1, FAKE, FAKE, FAKE, o, (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,
        "negative qlen");
  check(kt_rawint4_moe_workspace_bytes(&good, 1 << 30) == 0, "qlen x top_k beyond 2^31");
  check(kt_rawint4_moe_fwd(&good, 4, NULL, FAKE, FAKE, o, (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,
        "NULL inputs");
  check(kt_rawint4_moe_fwd(&good, 4, ODD, FAKE, FAKE, o, (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,
        "misaligned inputs");
  check(kt_rawint4_moe_fwd(&good, 4, FAKE, FAKE, FAKE, o, NULL, need, NULL) == KT_RAWINT4_EINVAL,
        "NULL workspace");
  check(kt_rawint4_moe_fwd(&good, 4, FAKE, FAKE, FAKE, o, (void*)ODD, need, NULL) == KT_RAWINT4_EINVAL,
        "misaligned workspace");
  check(kt_rawint4_moe_fwd(&good, 4, FAKE, FAKE, FAKE, o, (void*)FAKE, need - 256, NULL) == KT_RAWINT4_EWORKSPACE,
        "small workspace");
  check(kt_rawint4_moe_infer(&good, 4, FAKE, FAKE, FAKE, o, (void*)FAKE, 256, NULL) == KT_RAWINT4_EWORKSPACE,
        "small inference workspace");
  check(kt_rawint4_moe_bwd(&good, 4, FAKE, FAKE, FAKE, FAKE, o, NULL, g, g, g, g, g, g, 0, NAN, (void*)FAKE, need,
                           NULL) == KT_RAWINT4_EINVAL,
        "NaN grad_scale");
  check(kt_rawint4_moe_bwd(&good, 4, FAKE, FAKE, FAKE, FAKE, o, NULL, g, g, NULL, g, g, g, 0, 1.f, (void*)FAKE, need,
                           NULL) == KT_RAWINT4_EINVAL,
        "missing gradient buffer");
  check(kt_rawint4_moe_bwd_recompute(&good, 4, FAKE, FAKE, FAKE, NULL, o, NULL, g, g, g, g, g, g, 0, 1.f,
                                     (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,
        "recompute without grad_output");
  kt_rawint4_moe_layer big = layer(384, 8, 7168, 2048, 16);
  check(kt_rawint4_moe_infer_static(&big, 32, FAKE, FAKE, FAKE, o, NULL) == KT_RAWINT4_EWORKSPACE,
        "static call beyond its array");
  check(strlen(kt_rawint4_last_error()) > 0, "error message kept");

  check(kt_rawint4_unpack(FAKE, 4, 7, (int8_t*)FAKE, NULL) == KT_RAWINT4_EINVAL, "unpack with odd k");
  check(kt_rawint4_dequant(FAKE, FAKE, 4, 48, g, NULL) == KT_RAWINT4_EINVAL, "dequant with k not a multiple of 32");
  check(kt_rawint4_dequant(ODD, FAKE, 4, 64, g, NULL) == KT_RAWINT4_EINVAL, "dequant with misaligned codes");
  check(kt_rawint4_dequant_mxfp4(FAKE, FAKE, -1, 64, g, NULL) == KT_RAWINT4_EINVAL, "MXFP4 dequant with n < 0");
  check(kt_rawint4_group_workspace_bytes(4, 0, 8) == 0, "grouping size with top_k 0");
  int32_t* i32 = (int32_t*)FAKE;
  check(kt_rawint4_group(FAKE, 4, 2, 0, i32, i32, (void*)FAKE, 1u << 20, NULL) == KT_RAWINT4_EINVAL,
        "grouping with no experts");
  check(kt_rawint4_group(NULL, 4, 2, 8, i32, i32, (void*)FAKE, 1u << 20, NULL) == KT_RAWINT4_EINVAL,
        "grouping without ids");
  check(kt_rawint4_moe_diagnostics(NULL, 0, NULL, NULL, NULL) == KT_RAWINT4_EINVAL, "diagnostics without workspace");
  check(kt_rawint4_moe_diagnostics(FAKE, 8, NULL, NULL, NULL) == KT_RAWINT4_EWORKSPACE,
        "diagnostics with a short workspace");
  check(kt_rawint4_moe_saved_preactivations(&good, 4, FAKE, need, NULL, g, NULL) == KT_RAWINT4_EINVAL,
        "saved pre-activations without gate");
  printf("ok   argument errors\n");
}

static void metadata_and_profiling(void) {
  check(strcmp(kt_rawint4_weight_layout(), "compressed-tensors-rawint4-g32-v1") == 0, "weight layout name");
  float ms[32];
  int32_t launches[32];
  check(kt_rawint4_profile_enable(1) == KT_RAWINT4_OK, "profiling on");
  check(kt_rawint4_profile_read(ms, launches, 32) == 18, "profile read with nothing recorded");
  check(kt_rawint4_profile_read(ms, launches, 4) == KT_RAWINT4_EINVAL, "profile read into too few slots");
  check(kt_rawint4_profile_enable(0) == KT_RAWINT4_OK, "profiling off");
  int named = 0;
  for (int i = -2; i < 22; ++i) named += kt_rawint4_profile_phase_name(i)[0] != 0;
  check(named == 18, "phase names");
  printf("ok   metadata and profiling\n");
}

int main(void) {
  sweep_planner();
  argument_errors();
  metadata_and_profiling();
  printf("%d checks, %d failed\n", checks, fails);
  return fails ? 1 : 0;
}
