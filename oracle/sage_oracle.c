/*
 * sage_oracle.c — CPU oracle for microscaling-FP4 attention (forward pass).
 *
 * TEST INFRASTRUCTURE ONLY (see sage_oracle.h): used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library, with which it shares no code.
 * Plain C, FP32 arithmetic in the order the method states, exp in double rounded to FP32.
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math, no FMA contraction).
 *
 * Sources: SageAttention3 (arXiv 2505.11594): abstract; DeepTech article, section "solving two
 * obstacles and one difficulty" (1x16 microscaling of both matmuls; two-level quantisation of
 * P that first maps each token's values into [0, 448*6] and then applies FP4 microscaling;
 * FP4 has 15 representable values) and section "FP4 attention inference acceleration and
 * hardware implementation" (NVFP4 = E2M1 + 1x16 + E4M3 scale, MXFP4 = E2M1 + 1x32 + E8M0
 * scale; FP32 accumulator; P quantisation fused into the online softmax, which also yields
 * each row's maximum; P-tile columns permuted to match the accumulator layout, with the
 * matching reorder done in the quantisation kernel).
 *
 * Readings where the pages leave a step open (each one is a choice of this implementation):
 *  R1 E4M3 scale encoding: round to nearest, ties to even mantissa, values above 448 clamp
 *     to 448 (no NaN from overflow).
 *  R2 NVFP4 scale = E4M3(fl32(amax / 6)); 6 is the largest E2M1 magnitude, consistent with
 *     the [0, 448*6] range of the first level for P.
 *  R3 E2M1 code = the E2M1 value nearest to the exact quotient x / s, ties to the even code,
 *     magnitudes above 6 clamp to 6; the sign bit is the input's (so -0 and small negatives
 *     give code 0x8); s == 0 (all-zero block or E4M3 underflow) gives codes of +-0.
 *  R4 MXFP4 scale: the OCP Microscaling rule, 2^(floor(log2 amax) - 2) clamped to the E8M0
 *     range, byte 0 for an all-zero block; codes as R3 with s = that power of two.
 *  R5 Blocks lie along each matmul's contraction dimension: Q and K along D, V along tokens,
 *     P along keys.
 *  R6 Inside a 128-key tile, keys are grouped by the slot order of sage_oracle.h (slot
 *     32g+4t+i holds key 16t+4g+i); P and V blocks are runs of consecutive slots. This is
 *     the column permutation of P, with the matching reorder of the quantisation kernel.
 *  R7 The first level of P is per (row, key tile): E = exp(x - t) with t the tile's row
 *     maximum, P2 = fl32(2688 * E); the output weight of the tile is beta/2688 with
 *     beta = exp(t - m_new). Hence results depend on the tile size (128).
 *  R8 The softmax normaliser sums the unquantised E.
 *  R9 MXFP4 variant: E8M0 scales need no range fix, so the first level is dropped: P2 = E and
 *     the tile weight is beta.
 *  R10 Scores x = fl32(c * S), c = fl32(1/sqrt(D)) unless given; no smoothing of K.
 *  R11 Causal: key j is visible to query i iff j <= i; a (row, tile) with no visible key is
 *     skipped.
 *  R12 S sums block partials (each exact in FP32) in block order; l sums E in key order; the
 *     PV accumulation sums block partials in slot order.
 *  R13 Direct-P (the rit.work page on FP4 FlashAttention-4, section on what was done: scores
 *     go straight to the MXFP4 codes the second matmul consumes, and the normaliser is taken
 *     from the same rounded values): MXFP4 codes and scales of P exactly as R9, and the
 *     normaliser sums the dequantised P instead of E: per tile, the block partials
 *     scale * sum(code) in block order.
 *  R14 FP4 QK with FP8 P and V (the rit.work page on FP4 FlashAttention-4, section on what was
 *     done: in its distributed training P and V were kept in FP8, since every variant with
 *     MXFP4 for them diverged). Q and K are MXFP4 as R4. P and V are MXFP8: E4M3 elements in
 *     blocks of 32 consecutive slots (R5, R6) with one E8M0 scale 2^(floor(log2 amax) - 8)
 *     per block (the OCP Microscaling rule; 8 is the largest E4M3 exponent), byte 0 for an
 *     all-zero block; the element is the E4M3 value nearest the exact quotient x / scale,
 *     ties to the even code, magnitudes above 448 clamp to 448, sign bit the input's. As in
 *     R9, P2 = E with tile weight beta, and the normaliser sums E (R8).
 *
 * Slack (test aid, not part of the method): a P rounding decision whose input lies within
 * its window of its boundary may legitimately go either way in an implementation whose exp or
 * FP32 summation order differs by a few ulp. For each such decision the oracle adds the largest
 * change of the row's output that the other choice could cause. The window of element j of a
 * (row, tile) is relative, delta + ORC_SCORE_EPS * (|x_j| + |t|): delta covers exp (a few ulp)
 * and the FP32 sums of P; the second term covers the scores themselves, since S is summed in an
 * implementation-defined order (R12) and x = fl32(c S) is rounded, so x_j - t carries an
 * absolute error of a few ulp of |x_j| + |t|, which is E_j's relative error.
 */
#include "sage_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* 2^-20, i.e. 16 units of 2^-24: D/16 block partials summed in FP32 (at most 8 roundings), the
 * scale product and the scaling by c, each at most half an ulp of the score's magnitude */
#define ORC_SCORE_EPS (1.0 / 1048576.0)

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(1024 + m), e - 25);
  return sign ? -v : v;
}

float orc_e2m1_decode(unsigned code) {
  float v = E2M1_MAG[code & 7];
  return (code & 8) ? -v : v;
}

float orc_e4m3_decode(unsigned b) {
  unsigned s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  float v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexpf((float)m, -9);
  else v = ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
  return s ? -v : v;
}

float orc_e8m0_decode(unsigned b) {
  b &= 255;
  if (b == 255) return NAN;
  return ldexpf(1.0f, (int)b - 127);
}

/* R1: nearest of the 127 non-negative finite E4M3 values; ties to the even code. */
unsigned orc_e4m3_encode(float y) {
  unsigned best = 0;
  double bd = INFINITY;
  for (unsigned c = 0; c <= 126; ++c) {
    double d = fabs((double)y - (double)orc_e4m3_decode(c));
    if (d < bd || (d == bd && (c & 1u) == 0)) { bd = d; best = c; }
  }
  return best;
}

/* R3: distances |x| - v*s are exact in double wherever two candidates are close. */
unsigned orc_e2m1_quant(float x, float s) {
  unsigned sign = signbit(x) ? 8u : 0u;
  if (!(s > 0.0f)) return sign;
  double ax = fabs((double)x);
  unsigned best = 0;
  double bd = INFINITY;
  for (unsigned c = 0; c < 8; ++c) {
    double d = fabs(ax - (double)E2M1_MAG[c] * (double)s);
    if (d < bd || (d == bd && (c & 1u) == 0)) { bd = d; best = c; }
  }
  return sign | best;
}

void orc_e4m3_encode_many(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(y[i]);
}

void orc_e2m1_quant_many(const float* x, const float* s, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_quant(x[i], s[i]);
}

/* R4 */
unsigned orc_mx_scale(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  frexpf(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
  int X = (e - 1) - 2;
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  return (unsigned)(X + 127);
}

/* R14: E8M0 byte of an MXFP8 block */
unsigned orc_mx8_scale(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  frexpf(amax, &e);
  int X = (e - 1) - 8;
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  return (unsigned)(X + 127);
}

/* R14: E4M3 element of x with power-of-two scale s (x/s is exact in FP32 here) */
unsigned orc_e4m3_quant(float x, float s) {
  unsigned sign = signbit(x) ? 0x80u : 0u;
  if (!(s > 0.0f)) return sign;
  return sign | orc_e4m3_encode(fabsf(x) / s);
}

/* R6 */
int orc_slot_token(int slot) {
  int g = slot / 32, t = (slot % 32) / 4, i = slot % 4;
  return 16 * t + 4 * g + i;
}

void orc_quant_block_nv(const float* x, int n, uint8_t* codes, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(x[i]));
  float y = amax / 6.0f; /* R2: FP32 division */
  unsigned sb = orc_e4m3_encode(y);
  float s = orc_e4m3_decode(sb);
  for (int i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e2m1_quant(x[i], s);
  *scale = (uint8_t)sb;
}

void orc_quant_block_mx(const float* x, int n, uint8_t* codes, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(x[i]));
  unsigned sb = orc_mx_scale(amax);
  float s = orc_e8m0_decode(sb);
  for (int i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e2m1_quant(x[i], s);
  *scale = (uint8_t)sb;
}

void orc_quant_block_mx8(const float* x, int n, uint8_t* codes, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(x[i]));
  unsigned sb = orc_mx8_scale(amax);
  float s = orc_e8m0_decode(sb);
  for (int i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_quant(x[i], s);
  *scale = (uint8_t)sb;
}

static int valid_fmt(int fmt) { return fmt == ORC_NVFP4 || fmt == ORC_MXFP4 || fmt == ORC_MX4_PV8; }
static int blk_of(int fmt) { return fmt == ORC_NVFP4 ? 16 : 32; }
static int pv8(int fmt) { return fmt == ORC_MX4_PV8; }

/* block quantiser of P and V (Q and K of the R14 variant are MXFP4) */
static void quant_block(int fmt, const float* x, int n, uint8_t* codes, uint8_t* scale) {
  if (fmt == ORC_NVFP4) orc_quant_block_nv(x, n, codes, scale);
  else if (fmt == ORC_MXFP4) orc_quant_block_mx(x, n, codes, scale);
  else orc_quant_block_mx8(x, n, codes, scale);
}

/* value of one P or V element code, and the element quantiser with block scale s */
static float pv_val(int fmt, unsigned code) { return pv8(fmt) ? orc_e4m3_decode(code) : orc_e2m1_decode(code); }
static unsigned pv_quant(int fmt, float x, float s) { return pv8(fmt) ? orc_e4m3_quant(x, s) : orc_e2m1_quant(x, s); }

static void put_code(uint8_t* packed, int64_t pos, unsigned code) {
  uint8_t* b = packed + pos / 2;
  if (pos % 2 == 0) *b = (uint8_t)((*b & 0xF0u) | (code & 15u));
  else *b = (uint8_t)((*b & 0x0Fu) | ((code & 15u) << 4));
}

static unsigned get_code(const uint8_t* packed, int64_t pos) {
  uint8_t b = packed[pos / 2];
  return (pos % 2 == 0) ? (b & 15u) : (b >> 4);
}

/* Index of V's scale byte for channel d at slot position p of head bh: scales are stored tile
 * by tile, [B*H][Np/128][D][128/blk], so that one tile's scales for all channels are one run. */
static int64_t v_scale_index(int64_t bh, int d, int64_t p, int D, int64_t Np, int blk) {
  const int64_t nb = ORC_KV_TILE / blk;
  return ((bh * (Np / ORC_KV_TILE) + p / ORC_KV_TILE) * D + d) * nb + (p % ORC_KV_TILE) / blk;
}

/* V codes are stored tile by tile too, [B*H][Np/128][D][128 slots], a nibble per slot (a byte
 * in the R14 variant), so that one tile's codes for all channels are one run. Code index of
 * channel d at slot position p of head bh: */
static int64_t v_code_index(int64_t bh, int d, int64_t p, int D, int64_t Np) {
  return ((bh * (Np / ORC_KV_TILE) + p / ORC_KV_TILE) * D + d) * ORC_KV_TILE + p % ORC_KV_TILE;
}
static unsigned get_v_code(int fmt, const uint8_t* codes, int64_t i) { return pv8(fmt) ? codes[i] : get_code(codes, i); }

int orc_quant(int role, int fmt, const uint16_t* x, int B, int H, int N, int D,
              uint8_t* codes, uint8_t* scales) {
  if (!x || !codes || !scales || B <= 0 || H <= 0 || N <= 0) return ORC_ERR_ARG;
  if (D != 64 && D != 128) return ORC_ERR_ARG;
  if (!valid_fmt(fmt)) return ORC_ERR_ARG;
  const int blk = blk_of(fmt);
  /* rows (Q, K) and channel rows (V) are independent: OpenMP splits them, nothing else changes */
  if (role == ORC_ROLE_Q || role == ORC_ROLE_K) {
    /* R5: blocks along D; R14: MXFP4 */
    const int qk_fmt = pv8(fmt) ? ORC_MXFP4 : fmt;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < (int64_t)B * H * N; ++r) {
      float xb[32];
      uint8_t cb[32], sb;
      for (int b0 = 0; b0 < D; b0 += blk) {
        for (int u = 0; u < blk; ++u) xb[u] = orc_f16_to_f32(x[r * D + b0 + u]);
        quant_block(qk_fmt, xb, blk, cb, &sb);
        for (int u = 0; u < blk; ++u) put_code(codes + r * (D / 2), b0 + u, cb[u]);
        scales[r * (D / blk) + b0 / blk] = sb;
      }
    }
    return ORC_OK;
  }
  if (role != ORC_ROLE_V) return ORC_ERR_ARG;
  /* R5/R6: V blocks along tokens, in slot order inside each 128-token tile; zero padding */
  const int64_t Np = ((int64_t)N + ORC_KV_TILE - 1) / ORC_KV_TILE * ORC_KV_TILE;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t row = 0; row < (int64_t)B * H * D; ++row) {
    const int64_t bh = row / D;
    const int d = (int)(row % D);
    const uint16_t* xh = x + bh * N * D;
    float xb[32];
    uint8_t cb[32], sb;
    for (int64_t p0 = 0; p0 < Np; p0 += blk) {
      for (int u = 0; u < blk; ++u) {
        int64_t p = p0 + u;
        int64_t tok = (p / ORC_KV_TILE) * ORC_KV_TILE + orc_slot_token((int)(p % ORC_KV_TILE));
        xb[u] = tok < N ? orc_f16_to_f32(xh[tok * D + d]) : 0.0f;
      }
      quant_block(fmt, xb, blk, cb, &sb);
      for (int u = 0; u < blk; ++u) {
        const int64_t i = v_code_index(bh, d, p0 + u, D, Np);
        if (pv8(fmt)) codes[i] = cb[u];
        else put_code(codes, i, cb[u]);
      }
      scales[v_scale_index(bh, d, p0, D, Np, blk)] = sb;
    }
  }
  return ORC_OK;
}

/* R7/R9: one (row, tile) of P */
int orc_p_tile(int fmt, const float* x, const uint8_t* vis, float* E, uint8_t* codes,
               uint8_t* scales, float* t_out) {
  const int blk = blk_of(fmt);
  float t = -INFINITY;
  int any = 0;
  for (int s = 0; s < ORC_KV_TILE; ++s)
    if (vis[s]) { any = 1; t = fmaxf(t, x[s]); }
  if (!any) return 0;
  float P2[ORC_KV_TILE];
  for (int s = 0; s < ORC_KV_TILE; ++s) {
    E[s] = vis[s] ? (float)exp((double)x[s] - (double)t) : 0.0f;
    P2[s] = fmt == ORC_NVFP4 ? 2688.0f * E[s] : E[s];
  }
  for (int b = 0; b < ORC_KV_TILE / blk; ++b) quant_block(fmt, P2 + b * blk, blk, codes + b * blk, scales + b);
  *t_out = t;
  return 1;
}

static float scale_val(int fmt, unsigned b) { return fmt == ORC_NVFP4 ? orc_e4m3_decode(b) : orc_e8m0_decode(b); }

/* Largest |change| of the dequantised P block (weighted by vmax) that a different rounding
 * decision within its relative window could cause: element u's window is dlt[u], the block
 * scale's the largest window of the block. */
static double block_ambiguity(int fmt, const float* P2, const uint8_t* codes, unsigned sbyte,
                              const double* vmax, const uint8_t* exact, const double* dlt) {
  const int blk = blk_of(fmt);
  const float s = scale_val(fmt, sbyte);
  double worst_scale = 0.0, delta = 0.0;
  float amax = 0.0f;
  int has_exact = 0;
  for (int u = 0; u < blk; ++u) {
    amax = fmaxf(amax, P2[u]);
    has_exact |= exact[u];
    if (dlt[u] > delta) delta = dlt[u];
  }
  /* a block holding the exact tile maximum has its amax fixed (E = exp(0) = 1) */
  for (int k = -1; k <= 1 && !has_exact; k += 2) {
    unsigned alt;
    if (fmt == ORC_NVFP4) alt = orc_e4m3_encode((float)((double)(amax / 6.0f) * (1.0 + k * delta)));
    else if (fmt == ORC_MXFP4) alt = orc_mx_scale((float)((double)amax * (1.0 + k * delta)));
    else alt = orc_mx8_scale((float)((double)amax * (1.0 + k * delta)));
    if (alt == sbyte) continue;
    const float s2 = scale_val(fmt, alt);
    double a = 0.0;
    for (int u = 0; u < blk; ++u) {
      double v1 = (double)pv_val(fmt, codes[u]) * s;
      double v2 = (double)pv_val(fmt, pv_quant(fmt, P2[u], s2)) * s2;
      a += fabs(v2 - v1) * vmax[u];
    }
    if (a > worst_scale) worst_scale = a;
  }
  double elem = 0.0;
  for (int u = 0; u < blk; ++u) {
    if (P2[u] == 0.0f || exact[u]) continue;
    double worst = 0.0;
    for (int k = -1; k <= 1; k += 2) {
      unsigned c2 = pv_quant(fmt, (float)((double)P2[u] * (1.0 + k * dlt[u])), s);
      double dv = fabs((double)pv_val(fmt, c2) - (double)pv_val(fmt, codes[u])) * s;
      if (dv > worst) worst = dv;
    }
    elem += worst * vmax[u];
  }
  return worst_scale + elem;
}

static int attn_fwd_impl(int fmt, int direct_p, const uint8_t* q_codes, const uint8_t* q_scales,
                         const uint8_t* k_codes, const uint8_t* k_scales,
                         const uint8_t* v_codes, const uint8_t* v_scales,
                         int B, int H, int N, int D, int causal, float sm_scale,
                         const int64_t* rows, int64_t n_rows, float* out,
                         double* slack, double* lse, double* lse_slack, double delta, int nthreads) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales || !out) return ORC_ERR_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || (D != 64 && D != 128)) return ORC_ERR_ARG;
  if (!valid_fmt(fmt)) return ORC_ERR_ARG;
  const int64_t total = (int64_t)B * H * N;
  if (!rows) n_rows = total;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return ORC_ERR_ARG;

  const int blk = blk_of(fmt);
  const float c = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)D)); /* R10 */
  const int64_t Np = ((int64_t)N + ORC_KV_TILE - 1) / ORC_KV_TILE * ORC_KV_TILE;
  const int ntiles = (int)(Np / ORC_KV_TILE);
  const float Kp = fmt == ORC_NVFP4 ? 2688.0f : 1.0f;
  int slot_of_token[ORC_KV_TILE];
  for (int s = 0; s < ORC_KV_TILE; ++s) slot_of_token[orc_slot_token(s)] = s;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int64_t bh = row / N;
    const int i = (int)(row % N);
    const uint8_t* qc = q_codes + row * (D / 2);
    const uint8_t* qs = q_scales + row * (D / blk);
    float* O = (float*)calloc((size_t)D, sizeof(float));
    double* tile_t = (double*)malloc(sizeof(double) * (size_t)ntiles);
    double* tile_amb = (double*)malloc(sizeof(double) * (size_t)ntiles);
    double* tile_pamb = (double*)malloc(sizeof(double) * (size_t)ntiles);
    int ntile_used = 0;
    float m = -INFINITY, l = 0.0f;
    float x[ORC_KV_TILE], E[ORC_KV_TILE];
    /* Slack with Direct-P: a changed P value also moves the normaliser, so the output moves by
     * at most |dP| (|v| + max|O|) / l, and max|O| <= the head's largest |V-hat|. */
    double vhead = 0.0;
    if (slack && direct_p) {
      for (int d = 0; d < D; ++d) {
        for (int64_t p = 0; p < Np; ++p) {
          double v = fabs((double)pv_val(fmt, get_v_code(fmt, v_codes, v_code_index(bh, d, p, D, Np))) *
                          (double)scale_val(fmt, v_scales[v_scale_index(bh, d, p, D, Np, blk)]));
          if (v > vhead) vhead = v;
        }
      }
    }
    uint8_t vis[ORC_KV_TILE], pc[ORC_KV_TILE], ps[ORC_KV_TILE / 16];
    for (int kt = 0; kt < ntiles; ++kt) {
      if (causal && (int64_t)kt * ORC_KV_TILE > i) break; /* R11 */
      for (int s = 0; s < ORC_KV_TILE; ++s) {
        const int64_t j = (int64_t)kt * ORC_KV_TILE + orc_slot_token(s);
        vis[s] = (uint8_t)(j < N && (!causal || j <= i));
        x[s] = 0.0f;
        if (!vis[s]) continue;
        const uint8_t* kc = k_codes + (bh * N + j) * (D / 2);
        const uint8_t* ks = k_scales + (bh * N + j) * (D / blk);
        float S = 0.0f;
        for (int b = 0; b < D / blk; ++b) { /* R12: exact block partials, block order */
          float inner = 0.0f;
          for (int u = 0; u < blk; ++u) {
            const int k = b * blk + u;
            inner += orc_e2m1_decode(get_code(qc, k)) * orc_e2m1_decode(get_code(kc, k));
          }
          const float sc = scale_val(fmt, qs[b]) * scale_val(fmt, ks[b]); /* E8M0 for R14 too */
          S += sc * inner;
        }
        x[s] = c * S;
      }
      float t;
      if (!orc_p_tile(fmt, x, vis, E, pc, ps, &t)) continue;
      const float mn = fmaxf(m, t);
      const float alpha = (float)exp((double)m - (double)mn);
      const float beta = (float)exp((double)t - (double)mn);
      float sumE = 0.0f;
      if (!direct_p) {
        for (int o = 0; o < ORC_KV_TILE; ++o) sumE += E[slot_of_token[o]]; /* key order, R8 */
      } else {
        for (int b = 0; b < ORC_KV_TILE / blk; ++b) {                      /* R13 */
          float inner = 0.0f;
          for (int u = 0; u < blk; ++u) inner += pv_val(fmt, pc[b * blk + u]);
          sumE += scale_val(fmt, ps[b]) * inner;
        }
      }
      l = alpha * l + beta * sumE;
      const float w = beta / Kp;                                          /* R7/R9 */
      for (int d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int b = 0; b < ORC_KV_TILE / blk; ++b) {
          float inner = 0.0f;
          for (int u = 0; u < blk; ++u) {
            const int s = b * blk + u;
            inner += pv_val(fmt, pc[s]) *
                     pv_val(fmt, get_v_code(fmt, v_codes, v_code_index(bh, d, (int64_t)kt * ORC_KV_TILE + s, D, Np)));
          }
          const float sc = scale_val(fmt, ps[b]) *
                           scale_val(fmt, v_scales[v_scale_index(bh, d, (int64_t)kt * ORC_KV_TILE + b * blk, D, Np, blk)]);
          acc += sc * inner;
        }
        O[d] = alpha * O[d] + w * acc;
      }
      m = mn;
      if (slack || lse_slack) {
        double vmax[ORC_KV_TILE];
        float P2[ORC_KV_TILE];
        for (int s = 0; s < ORC_KV_TILE; ++s) {
          double mv = 0.0;
          for (int d = 0; d < D; ++d) {
            const int64_t p = (int64_t)kt * ORC_KV_TILE + s;
            double v = fabs((double)pv_val(fmt, get_v_code(fmt, v_codes, v_code_index(bh, d, p, D, Np))) *
                            (double)scale_val(fmt, v_scales[v_scale_index(bh, d, p, D, Np, blk)]));
            if (v > mv) mv = v;
          }
          vmax[s] = mv + vhead;
          P2[s] = fmt == ORC_NVFP4 ? 2688.0f * E[s] : E[s];
        }
        /* each element's decision window (header: delta plus the scores' own FP32 error) */
        double dlt[ORC_KV_TILE];
        for (int s = 0; s < ORC_KV_TILE; ++s)
          dlt[s] = delta + ORC_SCORE_EPS * (fabs((double)x[s]) + fabs((double)t));
        /* The tile maximum has E = exp(0) = 1 exactly in any implementation, unless another
         * visible key is within the window of it (or tied), in which case either may be the top. */
        uint8_t exact[ORC_KV_TILE];
        int top = -1;
        float second = 0.0f;
        for (int s = 0; s < ORC_KV_TILE; ++s) {
          exact[s] = 0;
          if (!vis[s]) continue;
          if (top < 0 && x[s] == t) top = s;
          else second = fmaxf(second, E[s]);
        }
        if (top >= 0 && (double)second < 1.0 - dlt[top]) exact[top] = 1;
        double amb = 0.0, pamb = 0.0;
        double ones[ORC_KV_TILE];
        for (int s = 0; s < ORC_KV_TILE; ++s) ones[s] = 1.0;
        for (int b = 0; b < ORC_KV_TILE / blk; ++b) {
          amb += block_ambiguity(fmt, P2 + b * blk, pc + b * blk, ps[b], vmax + b * blk, exact + b * blk,
                                 dlt + b * blk);
          /* with unit weights: how far the tile's sum of dequantised P can move (Direct-P lse) */
          if (direct_p)
            pamb += block_ambiguity(fmt, P2 + b * blk, pc + b * blk, ps[b], ones, exact + b * blk, dlt + b * blk);
        }
        tile_t[ntile_used] = t;
        tile_amb[ntile_used] = amb;
        tile_pamb[ntile_used] = pamb;
        ++ntile_used;
      }
    }
    float* o = out + r * D;
    for (int d = 0; d < D; ++d) o[d] = O[d] / l;
    if (slack) {
      double sl = 0.0;
      for (int u = 0; u < ntile_used; ++u) sl += exp(tile_t[u] - (double)m) * tile_amb[u];
      slack[r] = sl / ((double)Kp * (double)l);
    }
    /* the row's log-sum-exp: l sums E (Direct-P: the dequantised P) in the frame of m */
    if (lse) lse[r] = (double)m + log((double)l);
    if (lse_slack) {
      /* |d ln l| <= |dl| / l; only Direct-P's l depends on rounding decisions */
      double sl = 0.0;
      for (int u = 0; u < ntile_used; ++u) sl += exp(tile_t[u] - (double)m) * tile_pamb[u];
      lse_slack[r] = sl / (double)l;
    }
    free(O);
    free(tile_t);
    free(tile_amb);
    free(tile_pamb);
  }
  return ORC_OK;
}

int orc_attn_fwd(int fmt, const uint8_t* q_codes, const uint8_t* q_scales,
                 const uint8_t* k_codes, const uint8_t* k_scales,
                 const uint8_t* v_codes, const uint8_t* v_scales,
                 int B, int H, int N, int D, int causal, float sm_scale,
                 const int64_t* rows, int64_t n_rows, float* out,
                 double* slack, double delta, int nthreads) {
  return attn_fwd_impl(fmt, 0, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, B, H, N, D, causal,
                       sm_scale, rows, n_rows, out, slack, NULL, NULL, delta, nthreads);
}

int orc_attn_fwd_direct_p(const uint8_t* q_codes, const uint8_t* q_scales,
                          const uint8_t* k_codes, const uint8_t* k_scales,
                          const uint8_t* v_codes, const uint8_t* v_scales,
                          int B, int H, int N, int D, int causal, float sm_scale,
                          const int64_t* rows, int64_t n_rows, float* out,
                          double* slack, double delta, int nthreads) {
  return attn_fwd_impl(ORC_MXFP4, 1, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, B, H, N, D,
                       causal, sm_scale, rows, n_rows, out, slack, NULL, NULL, delta, nthreads);
}

int orc_attn_fwd_lse(int fmt, int direct_p, const uint8_t* q_codes, const uint8_t* q_scales,
                     const uint8_t* k_codes, const uint8_t* k_scales,
                     const uint8_t* v_codes, const uint8_t* v_scales,
                     int B, int H, int N, int D, int causal, float sm_scale,
                     const int64_t* rows, int64_t n_rows, float* out, double* lse,
                     double* slack, double* lse_slack, double delta, int nthreads) {
  if (!lse || (direct_p && fmt != ORC_MXFP4)) return ORC_ERR_ARG;
  return attn_fwd_impl(fmt, direct_p ? 1 : 0, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, B, H, N,
                       D, causal, sm_scale, rows, n_rows, out, slack, lse, lse_slack, delta, nthreads);
}

int orc_attn_ref_f64(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int B, int H, int N, int D, int causal, double sm_scale,
                     const int64_t* rows, int64_t n_rows, double* out, int nthreads) {
  if (!q || !k || !v || !out || B <= 0 || H <= 0 || N <= 0 || D <= 0) return ORC_ERR_ARG;
  const int64_t total = (int64_t)B * H * N;
  if (!rows) n_rows = total;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return ORC_ERR_ARG;
  const double c = sm_scale > 0.0 ? sm_scale : 1.0 / sqrt((double)D);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int64_t bh = row / N;
    const int i = (int)(row % N);
    const int nk = causal ? i + 1 : N;
    double* sc = (double*)malloc(sizeof(double) * (size_t)nk);
    double mx = -INFINITY;
    for (int j = 0; j < nk; ++j) {
      double s = 0.0;
      for (int d = 0; d < D; ++d)
        s += (double)orc_f16_to_f32(q[row * D + d]) * (double)orc_f16_to_f32(k[(bh * N + j) * D + d]);
      sc[j] = c * s;
      if (sc[j] > mx) mx = sc[j];
    }
    double den = 0.0;
    for (int j = 0; j < nk; ++j) { sc[j] = exp(sc[j] - mx); den += sc[j]; }
    double* o = out + r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int j = 0; j < nk; ++j)
      for (int d = 0; d < D; ++d) o[d] += sc[j] * (double)orc_f16_to_f32(v[(bh * N + j) * D + d]);
    for (int d = 0; d < D; ++d) o[d] /= den;
    free(sc);
  }
  return ORC_OK;
}
