/* Driver for the sanitizer build of the oracle (built by tests/test_oracle_sanitized.py with
 * gcc -fsanitize=address,undefined): calls every entry point of sage_oracle.h on small seeded
 * inputs that include a ragged last tile, every format and role, causal and not, explicit
 * sm_scale, selected rows and the slack, and checks that each call succeeds and returns finite
 * values. Any out-of-bounds access, leak or undefined behaviour aborts with a sanitizer report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/sage_oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double unif(void) {
  st += 0x9E3779B97F4A7C15ull;
  uint64_t z = st;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

/* fp16 bits of a value in [-4, 4) with 8 significant bits (exactly representable) */
static uint16_t rnd_f16(void) {
  double x = (unif() * 8.0 - 4.0);
  int e;
  frexp(x, &e);
  x = ldexp(round(ldexp(x, 8 - e)), e - 8);
  if (x == 0.0) return 0;
  uint16_t s = x < 0 ? 0x8000 : 0;
  x = fabs(x);
  int ex;
  double m = frexp(x, &ex); /* x = m 2^ex, m in [0.5, 1) */
  int E = ex - 1 + 15;
  if (E <= 0) return s;
  uint16_t mant = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
  return (uint16_t)(s | (E << 10) | mant);
}

#define CHECK(cond, what)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "check failed: %s\n", what);         \
      return 1;                                            \
    }                                                      \
  } while (0)

static int finite_all(const float* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

static int run_case(int fmt, int B, int H, int N, int D) {
  const int64_t el = (int64_t)B * H * N * D;
  const int blk = fmt == ORC_NVFP4 ? 16 : 32;
  const int64_t Np = ((int64_t)N + ORC_KV_TILE - 1) / ORC_KV_TILE * ORC_KV_TILE;
  uint16_t* x[3];
  for (int t = 0; t < 3; ++t) {
    x[t] = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)el);
    for (int64_t i = 0; i < el; ++i) x[t][i] = rnd_f16();
  }
  const int64_t qk_codes = el / 2, qk_scales = el / blk;
  const int64_t v_codes = (int64_t)B * H * D * (fmt == ORC_MX4_PV8 ? Np : Np / 2);
  const int64_t v_scales = (int64_t)B * H * D * (Np / blk);
  uint8_t* c[3];
  uint8_t* s[3];
  for (int t = 0; t < 3; ++t) {
    c[t] = (uint8_t*)malloc((size_t)(t == 2 ? v_codes : qk_codes));
    s[t] = (uint8_t*)malloc((size_t)(t == 2 ? v_scales : qk_scales));
    CHECK(orc_quant(t, fmt, x[t], B, H, N, D, c[t], s[t]) == ORC_OK, "quant");
  }
  const int64_t rows_all = (int64_t)B * H * N;
  /* all rows: [B,H,N,D]; three selected rows: [3, D] */
  float* out = (float*)malloc(sizeof(float) * (size_t)(el > 3 * D ? el : 3 * D));
  double* slack = (double*)malloc(sizeof(double) * (size_t)(rows_all > 3 ? rows_all : 3));
  double* lse = (double*)malloc(sizeof(double) * (size_t)rows_all);
  double* lse_slack = (double*)malloc(sizeof(double) * (size_t)rows_all);
  for (int causal = 0; causal < 2; ++causal) {
    CHECK(orc_attn_fwd(fmt, c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, D, causal, 0.0f, NULL, 0, out,
                       slack, 1.0 / 16384.0, 0) == ORC_OK, "attn_fwd");
    CHECK(finite_all(out, el), "attn_fwd finite");
    CHECK(orc_attn_fwd_lse(fmt, 0, c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, D, causal, 0.3f, NULL, 0, out,
                           lse, slack, lse_slack, 1.0 / 16384.0, 0) == ORC_OK, "attn_fwd_lse");
    CHECK(finite_all(out, el), "attn_fwd_lse finite");
    if (fmt == ORC_MXFP4) {
      CHECK(orc_attn_fwd_direct_p(c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, D, causal, 0.0f, NULL, 0, out,
                                  slack, 1.0 / 16384.0, 0) == ORC_OK, "direct_p");
      CHECK(orc_attn_fwd_lse(fmt, 1, c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, D, causal, 0.0f, NULL, 0,
                             out, lse, slack, lse_slack, 1.0 / 16384.0, 0) == ORC_OK, "direct_p lse");
    }
    int64_t rows[3] = {0, rows_all - 1, rows_all / 2};
    CHECK(orc_attn_fwd(fmt, c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, D, causal, 0.0f, rows, 3, out,
                       slack, 1.0 / 16384.0, 0) == ORC_OK, "attn_fwd rows");
    double* ref = (double*)malloc(sizeof(double) * (size_t)el);
    CHECK(orc_attn_ref_f64(x[0], x[1], x[2], B, H, N, D, causal, 0.0, NULL, 0, ref, 0) == ORC_OK, "ref");
    free(ref);
  }
  /* rejected arguments return an error and touch nothing */
  CHECK(orc_attn_fwd(fmt, c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, 96, 0, 0.0f, NULL, 0, out, NULL,
                     1.0 / 16384.0, 0) != ORC_OK, "bad D");
  int64_t bad_row = rows_all;
  CHECK(orc_attn_fwd(fmt, c[0], s[0], c[1], s[1], c[2], s[2], B, H, N, D, 0, 0.0f, &bad_row, 1, out, NULL,
                     1.0 / 16384.0, 0) != ORC_OK, "bad row");
  for (int t = 0; t < 3; ++t) { free(x[t]); free(c[t]); free(s[t]); }
  free(out); free(slack); free(lse); free(lse_slack);
  return 0;
}

int main(void) {
  /* one P tile with a partly visible row */
  float xs[ORC_KV_TILE], E[ORC_KV_TILE], t;
  uint8_t vis[ORC_KV_TILE], codes[ORC_KV_TILE], scales[ORC_KV_TILE / 16];
  for (int i = 0; i < ORC_KV_TILE; ++i) { xs[i] = (float)(unif() * 6.0 - 3.0); vis[i] = (uint8_t)(i < 77); }
  for (int fmt = 0; fmt < 3; ++fmt) CHECK(orc_p_tile(fmt, xs, vis, E, codes, scales, &t) == 1, "p_tile");
  const int shapes[][4] = {{1, 2, 130, 64}, {2, 1, 77, 128}, {1, 1, 1, 64}};
  for (int fmt = 0; fmt < 3; ++fmt)
    for (int k = 0; k < 3; ++k)
      if (run_case(fmt, shapes[k][0], shapes[k][1], shapes[k][2], shapes[k][3])) {
        fprintf(stderr, "case fmt %d shape %d failed\n", fmt, k);
        return 1;
      }
  printf("sanitized oracle: all entry points ok\n");
  return 0;
}
