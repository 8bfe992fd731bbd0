/* Plain-C client of include/sage_fp4.h: compiles the header as C99 and exercises every entry point
 * that needs no GPU (version, tile, slot order, size helpers, status strings) plus the host-side
 * validation of the launching entry points, which returns before anything is enqueued. Built and
 * run by tests/test_c_header.py; prints "C ABI OK" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sage_fp4.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  /* never dereferenced: every call below fails validation first */
  void* fake = (void*)(uintptr_t)0x10000;
  void* mis = (void*)(uintptr_t)0x10008;
  int s;

  CHECK(sage_fp4_version() >= 300);
  CHECK(sage_fp4_kv_tile() == 128);
  {
    int seen[128];
    memset(seen, 0, sizeof seen);
    for (s = 0; s < 128; ++s) {
      int t = sage_fp4_slot_token(s);
      CHECK(t >= 0 && t < 128);
      if (t >= 0 && t < 128) seen[t]++;
      CHECK(t == 16 * ((s % 32) / 4) + 4 * (s / 32) + s % 4);
    }
    for (s = 0; s < 128; ++s) CHECK(seen[s] == 1);
    CHECK(sage_fp4_slot_token(128) == -1 && sage_fp4_slot_token(-1) == -1);
  }

  /* layouts: B=2 H=3 N=300 D=128, Np = 384 */
  CHECK(sage_fp4_codes_bytes(SAGE_ROLE_Q, SAGE_FMT_NVFP4, 2, 3, 300, 128) == (size_t)2 * 3 * 300 * 64);
  CHECK(sage_fp4_scales_bytes(SAGE_ROLE_K, SAGE_FMT_NVFP4, 2, 3, 300, 128) == (size_t)2 * 3 * 300 * 8);
  CHECK(sage_fp4_scales_bytes(SAGE_ROLE_K, SAGE_FMT_MXFP4, 2, 3, 300, 128) == (size_t)2 * 3 * 300 * 4);
  CHECK(sage_fp4_codes_bytes(SAGE_ROLE_V, SAGE_FMT_MXFP4, 2, 3, 300, 128) == (size_t)2 * 3 * 128 * 192);
  CHECK(sage_fp4_codes_bytes(SAGE_ROLE_V, SAGE_FMT_MX4_PV8, 2, 3, 300, 128) == (size_t)2 * 3 * 128 * 384);
  CHECK(sage_fp4_scales_bytes(SAGE_ROLE_V, SAGE_FMT_MX4_PV8, 2, 3, 300, 128) == (size_t)2 * 3 * 128 * 12);
  CHECK(sage_fp4_codes_bytes(SAGE_ROLE_Q, SAGE_FMT_NVFP4, 2, 3, 300, 96) == 0);
  CHECK(sage_fp4_codes_bytes(SAGE_ROLE_Q, 7, 2, 3, 300, 128) == 0);

  /* validation before any launch */
  CHECK(sage_fp4_quant(SAGE_ROLE_V, SAGE_FMT_NVFP4, NULL, 1, 1, 16, 64, fake, fake, NULL) == SAGE_ERR_NULL);
  CHECK(sage_fp4_quant(SAGE_ROLE_V, SAGE_FMT_NVFP4, fake, 1, 1, 16, 80, fake, fake, NULL) == SAGE_ERR_HEAD_DIM);
  CHECK(sage_fp4_quant(SAGE_ROLE_V, SAGE_FMT_NVFP4, fake, 1, 1, 0, 64, fake, fake, NULL) == SAGE_ERR_SHAPE);
  CHECK(sage_fp4_quant(SAGE_ROLE_V, SAGE_FMT_NVFP4, mis, 1, 1, 16, 64, fake, fake, NULL) == SAGE_ERR_ALIGN);
  CHECK(sage_fp4_quant(9, SAGE_FMT_NVFP4, fake, 1, 1, 16, 64, fake, fake, NULL) == SAGE_ERR_ENUM);
  CHECK(sage_fp4_attn_fwd(SAGE_FMT_MX4_PV8, fake, fake, fake, fake, fake, NULL, 1, 1, 16, 64, 0, 0.0f, fake,
                          SAGE_OUT_F32, NULL) == SAGE_ERR_NULL);
  CHECK(sage_fp4_attn_fwd(SAGE_FMT_NVFP4, fake, fake, fake, fake, fake, fake, 1, 1, 16, 64, 1, 0.0f, fake, 5,
                          NULL) == SAGE_ERR_ENUM);
  CHECK(sage_fp4_attn_fwd(SAGE_FMT_MXFP4, fake, fake, fake, fake, fake, fake, 70000, 1, 16, 64, 0, 0.0f, fake,
                          SAGE_OUT_F16, NULL) == SAGE_ERR_SHAPE);
  CHECK(sage_fp4_attn_fwd_direct_p(fake, fake, fake, fake, fake, fake, 1, 1, 16, 64, 0, 0.0f, mis, SAGE_OUT_F16,
                                   NULL) == SAGE_ERR_ALIGN);
  CHECK(sage_fp4_attn_fwd_lse(SAGE_FMT_NVFP4, 0, fake, fake, fake, fake, fake, fake, 1, 1, 16, 64, 0, 0.0f, fake,
                              SAGE_OUT_F32, NULL, NULL) == SAGE_ERR_NULL);
  CHECK(sage_fp4_attn_fwd_lse(SAGE_FMT_NVFP4, 1, fake, fake, fake, fake, fake, fake, 1, 1, 16, 64, 0, 0.0f, fake,
                              SAGE_OUT_F32, (float*)fake, NULL) == SAGE_ERR_ENUM);
  CHECK(sage_fp4_attn_fwd_lse(SAGE_FMT_MXFP4, 1, fake, fake, fake, fake, fake, fake, 1, 1, 16, 64, 0, 0.0f, fake,
                              SAGE_OUT_F32, (float*)mis, NULL) == SAGE_ERR_ALIGN);
  /* backward: workspace size (B=2 H=3 N=300 D=128: Np64 = 320, 5 blocks) and validation */
  {
    const size_t qh = 2 * 3 * 300 * 128 * 2, i8 = 2 * 3 * 128 * 320, sc = 2 * 3 * 128 * 5 * 4, dl = 2 * 3 * 320 * 4;
#define A256(x) (((x) + 255) / 256 * 256)
    CHECK(sage_fp4_attn_bwd_workspace_bytes(2, 3, 300, 128) ==
          2 * A256(qh) + 3 * A256(i8) + 3 * A256(sc) + 2 * A256(dl));
#undef A256
    CHECK(sage_fp4_attn_bwd_workspace_bytes(2, 3, 300, 96) == 0);
    size_t need = sage_fp4_attn_bwd_workspace_bytes(1, 1, 16, 64);
    CHECK(need > 0);
    CHECK(sage_fp4_attn_bwd(SAGE_FMT_NVFP4, fake, fake, fake, fake, fake, fake, fake, (const float*)fake, 1, 1, 16,
                            64, 0, 0.0f, fake, fake, fake, SAGE_OUT_F32, fake, need - 1, NULL) == SAGE_ERR_WORKSPACE);
    CHECK(sage_fp4_attn_bwd(SAGE_FMT_NVFP4, fake, fake, fake, fake, fake, fake, NULL, (const float*)fake, 1, 1, 16,
                            64, 0, 0.0f, fake, fake, fake, SAGE_OUT_F32, fake, need, NULL) == SAGE_ERR_NULL);
    CHECK(sage_fp4_attn_bwd(SAGE_FMT_NVFP4, fake, fake, fake, fake, fake, fake, fake, (const float*)fake, 1, 1, 16,
                            64, 0, 0.0f, fake, fake, fake, SAGE_OUT_F32, NULL, need, NULL) == SAGE_ERR_NULL);
    CHECK(sage_fp4_attn_bwd(SAGE_FMT_MXFP4, fake, fake, fake, fake, fake, fake, fake, (const float*)fake, 1, 1, 16,
                            64, 0, 0.0f, fake, mis, fake, SAGE_OUT_F16, fake, need, NULL) == SAGE_ERR_ALIGN);
    CHECK(sage_fp4_attn_bwd(3, fake, fake, fake, fake, fake, fake, fake, (const float*)fake, 1, 1, 16, 64, 0, 0.0f,
                            fake, fake, fake, SAGE_OUT_F16, fake, need, NULL) == SAGE_ERR_ENUM);
    CHECK(sage_fp4_attn_bwd(SAGE_FMT_MX4_PV8, fake, fake, fake, fake, fake, fake, fake, (const float*)fake, 1, 1, 16,
                            64, 0, 0.0f, fake, fake, fake, 2, fake, need, NULL) == SAGE_ERR_ENUM);
    CHECK(sage_fp4_attn_bwd(SAGE_FMT_NVFP4, fake, fake, fake, fake, fake, fake, fake, (const float*)fake, 1, 1, 16,
                            80, 0, 0.0f, fake, fake, fake, SAGE_OUT_F32, fake, need, NULL) == SAGE_ERR_HEAD_DIM);
  }
  /* dequantised K/V: buffer size (Np = 384) and validation */
  {
    CHECK(sage_fp4_kv16_bytes(2, 3, 300, 128) == (size_t)4 * 2 * 3 * 384 * 128);
    CHECK(sage_fp4_kv16_bytes(2, 3, 300, 96) == 0);
    size_t need = sage_fp4_kv16_bytes(1, 1, 16, 64);
    CHECK(sage_fp4_kv16_prep(fake, fake, fake, fake, 1, 1, 16, 64, fake, need - 1, NULL) == SAGE_ERR_WORKSPACE);
    CHECK(sage_fp4_kv16_prep(fake, fake, fake, NULL, 1, 1, 16, 64, fake, need, NULL) == SAGE_ERR_NULL);
    CHECK(sage_fp4_kv16_prep(fake, fake, fake, fake, 1, 1, 16, 64, mis, need, NULL) == SAGE_ERR_ALIGN);
    CHECK(sage_fp4_quant_kv16(SAGE_ROLE_Q, fake, 1, 1, 16, 64, fake, fake, fake, need, NULL) == SAGE_ERR_ENUM);
    CHECK(sage_fp4_quant_kv16(SAGE_ROLE_K, fake, 1, 1, 16, 64, fake, fake, fake, need - 1, NULL) == SAGE_ERR_WORKSPACE);
    CHECK(sage_fp4_quant_kv16(SAGE_ROLE_V, fake, 1, 1, 16, 64, fake, fake, NULL, need, NULL) == SAGE_ERR_NULL);
    CHECK(sage_fp4_attn_fwd_kv16(fake, fake, fake, need - 1, 1, 1, 16, 64, 0, 0.0f, fake, SAGE_OUT_F32, NULL, NULL) ==
          SAGE_ERR_WORKSPACE);
    CHECK(sage_fp4_attn_fwd_kv16(fake, fake, fake, need, 1, 1, 16, 64, 0, 0.0f, fake, 3, NULL, NULL) == SAGE_ERR_ENUM);
    CHECK(sage_fp4_attn_fwd_kv16(fake, fake, fake, need, 1, 1, 16, 64, 0, 0.0f, fake, SAGE_OUT_F16, (float*)mis,
                                 NULL) == SAGE_ERR_ALIGN);
  }
  for (s = -7; s <= 0; ++s) CHECK(sage_fp4_status_string(s) != NULL && strlen(sage_fp4_status_string(s)) > 0);
  CHECK(strcmp(sage_fp4_status_string(SAGE_ERR_WORKSPACE), "unknown status") != 0);
  CHECK(strcmp(sage_fp4_status_string(SAGE_OK), "ok") == 0);

  if (failures) return 1;
  printf("C ABI OK\n");
  return 0;
}
