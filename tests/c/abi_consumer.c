/*
 * A plain C consumer of the library's C ABI: compiled with gcc against
 * include/kt_rawint4.h and linked to libkt_rawint4.so.  It only makes calls
 * that the host checks answer before any GPU work (sizes, argument errors,
 * metadata), so it runs on a machine without a GPU.  Prints one line per check
 * and exits nonzero on the first failure.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "kt_rawint4.h"

#define FAKE ((const void*)(uintptr_t)(1u << 20)) /* 256-byte aligned, never dereferenced */

static int fails = 0;
static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++fails;
}

static kt_rawint4_moe_layer layer(void) {
  kt_rawint4_moe_layer L;
  memset(&L, 0, sizeof L);
  L.num_experts = 8;
  L.top_k = 2;
  L.hidden = 512;
  L.intermediate = 384;
  L.rank = 8;
  L.alpha = 16.f;
  L.swiglu_limit = 2.f;
  L.gate_packed = L.up_packed = L.down_packed = (const uint8_t*)FAKE;
  L.gate_scale = L.up_scale = L.down_scale = (const uint16_t*)FAKE;
  L.gate_lora_a = L.gate_lora_b = L.up_lora_a = L.up_lora_b = L.down_lora_a = L.down_lora_b = (const float*)FAKE;
  return L; /* weight_format 0: RAWINT4 */
}

int main(void) {
  kt_rawint4_moe_layer L = layer();
  const size_t small = kt_rawint4_moe_workspace_bytes(&L, 5), big = kt_rawint4_moe_workspace_bytes(&L, 500);
  check(small > 0 && big > small && small % 256 == 0, "training workspace grows with tokens");
  const size_t inf = kt_rawint4_moe_infer_workspace_bytes(&L, 500);
  check(inf > 0 && inf < big, "inference workspace is smaller");

  kt_rawint4_moe_layer base = layer();
  base.gate_lora_a = base.gate_lora_b = base.up_lora_a = base.up_lora_b = base.down_lora_a = base.down_lora_b = NULL;
  base.rank = 0;
  check(kt_rawint4_moe_infer_workspace_bytes(&base, 500) > 0, "frozen base alone accepted by inference");
  check(kt_rawint4_moe_workspace_bytes(&base, 500) == 0 && strstr(kt_rawint4_last_error(), "rank") != NULL,
        "frozen base alone rejected by training");

  kt_rawint4_moe_layer bad = layer();
  bad.hidden = 500;
  check(kt_rawint4_moe_fwd(&bad, 4, FAKE, FAKE, FAKE, (uint16_t*)FAKE, (void*)FAKE, 1u << 30, NULL) ==
            KT_RAWINT4_EINVAL,
        "hidden not a multiple of 32 rejected");
  bad = layer();
  bad.weight_format = 7;
  check(kt_rawint4_moe_workspace_bytes(&bad, 4) == 0 && strstr(kt_rawint4_last_error(), "weight_format"),
        "unknown weight format rejected");
  kt_rawint4_moe_layer mx = layer();
  mx.weight_format = KT_RAWINT4_FORMAT_MXFP4;
  check(kt_rawint4_moe_workspace_bytes(&mx, 4) == kt_rawint4_moe_workspace_bytes(&L, 4), "MXFP4 layer accepted");

  const size_t need = kt_rawint4_moe_workspace_bytes(&L, 4);
  check(kt_rawint4_moe_fwd(&L, 4, FAKE, FAKE, FAKE, (uint16_t*)FAKE, (void*)FAKE, need - 256, NULL) ==
            KT_RAWINT4_EWORKSPACE,
        "small workspace rejected");
  float* g = (float*)FAKE;
  check(kt_rawint4_moe_bwd(&L, 4, FAKE, FAKE, FAKE, FAKE, (uint16_t*)FAKE, NULL, g, g, g, g, g, g, 0, NAN,
                           (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL &&
            strstr(kt_rawint4_last_error(), "grad_scale"),
        "non-finite grad_scale rejected");
  check(kt_rawint4_moe_bwd_recompute(&L, 4, FAKE, FAKE, FAKE, FAKE, (uint16_t*)FAKE, NULL, g, g, g, g, g, NULL, 0,
                                     1.f, (void*)FAKE, need, NULL) == KT_RAWINT4_EINVAL,
        "missing gradient buffer rejected by the recompute backward");
  check(strcmp(kt_rawint4_weight_layout(), "compressed-tensors-rawint4-g32-v1") == 0, "weight layout name");
  check(kt_rawint4_dequant_mxfp4(FAKE, FAKE, 4, 48, (float*)FAKE, NULL) == KT_RAWINT4_EINVAL,
        "MXFP4 dequant hook checks k");
  return fails ? 1 : 0;
}
