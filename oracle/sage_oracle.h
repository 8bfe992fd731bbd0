/*
 * sage_oracle.h — CPU oracle for microscaling-FP4 attention (forward pass).
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow reference that the GPU library is checked
 * against. Only the test suite, the package's smoke check and the CPU-baseline leg of the
 * benchmark may load it. The GPU library never links, imports or calls it, and it shares no
 * code, header, table or helper with the GPU library.
 *
 * What it computes (SageAttention3, "Microscaling FP4 Attention for Inference and An
 * Exploration of 8-Bit Training", arXiv 2505.11594; the DeepTech article on it, sections
 * "two obstacles and one difficulty" and "FP4 attention inference acceleration"):
 *   - NVFP4: E2M1 values in 1x16 blocks with one E4M3 scale per block;
 *     MXFP4: E2M1 values in 1x32 blocks with one E8M0 scale per block.
 *   - Q and K are quantised along the head dimension D, V along tokens (the contraction
 *     dimension of P.V); both matmuls use FP4 operands and FP32 accumulation.
 *   - an online softmax over key tiles of ORC_KV_TILE keys, in which P is quantised in two
 *     levels: per (row, tile) the values are scaled into [0, 448*6], then 1x16 FP4
 *     microscaling is applied.
 * Every arithmetic step is written out in FP32 in the order the method states; exp is
 * evaluated in double and rounded to FP32. Readings of steps the pages leave open are listed
 * in the header of sage_oracle.c.
 *
 * Parity pins: every function here is pinned by the CPU tests (codec tables against the torch
 * float8 codecs, closed-form tie cases, lossless special cases of the attention, one-hot
 * attention at every slot position, the FP64 unquantised reference against torch SDPA).
 *
 * Layouts (all row-major, contiguous, bytes unless stated):
 *   x (fp16 bits)        [B,H,N,D]
 *   Q/K codes            [B,H,N,D/2]      element 2i in the low nibble of byte i
 *   Q/K scales           [B,H,N,D/16] (E4M3) or [B,H,N,D/32] (E8M0)
 *   V codes              [B,H,Np/128,D,64]  tile by tile, tokens in slot order inside each
 *                        128-token tile (slot 2i in the low nibble of byte i of the channel's 64)
 *   V scales             [B,H,Np/128,D,8] or [B,H,Np/128,D,4]   tile by tile as well: one
 *                        128-token tile's codes, and its scales, for every channel are one run
 *   Np = ceil(N/128)*128; token positions >= N are zero.
 * ORC_MX4_PV8 (FP4 QK, FP8 PV; reading R14 in sage_oracle.c): Q/K codes and scales as MXFP4;
 *   V codes [B,H,Np/128,D,128] one E4M3 byte per element (slot order), V scales
 *   [B,H,Np/128,D,4] E8M0.
 * Slot order inside a 128-token tile: slot s = 32g + 4t + i holds token 16t + 4g + i
 * (g in 0..3, t in 0..7, i in 0..3). Blocks of P and of V are consecutive slots.
 */
#ifndef SAGE_ORACLE_H
#define SAGE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_KV_TILE 128

enum { ORC_NVFP4 = 0, ORC_MXFP4 = 1, ORC_MX4_PV8 = 2 };
enum { ORC_ROLE_Q = 0, ORC_ROLE_K = 1, ORC_ROLE_V = 2 };
enum { ORC_OK = 0, ORC_ERR_ARG = -1 };

/* ---- element codecs ---- */
float orc_f16_to_f32(uint16_t h);                /* exact */
float orc_e2m1_decode(unsigned code);            /* 4-bit code -> value (bit 3 = sign) */
float orc_e4m3_decode(unsigned byte);            /* OCP E4M3 (fn): bias 7, max 448, NaN 0x7F/0xFF */
float orc_e8m0_decode(unsigned byte);            /* 2^(byte-127); 0xFF = NaN */
unsigned orc_e4m3_encode(float y);               /* y >= 0 finite: nearest E4M3, ties to even, clamp 448 */
unsigned orc_e2m1_quant(float x, float s);       /* nearest E2M1 to the exact x/s, ties to even, clamp 6 */
unsigned orc_mx_scale(float amax);               /* E8M0 byte: floor(log2 amax) - 2, clamped; 0 if amax == 0 */
unsigned orc_mx8_scale(float amax);              /* E8M0 byte: floor(log2 amax) - 8, clamped; 0 if amax == 0 */
unsigned orc_e4m3_quant(float x, float s);       /* sign | nearest E4M3 to |x|/s (s a power of two), ties even, clamp 448 */
int orc_slot_token(int slot);                    /* token offset held by slot (0..127) */
/* bulk forms of the two encoders (loops over the scalar functions above) */
void orc_e4m3_encode_many(const float* y, int64_t n, uint8_t* out);
void orc_e2m1_quant_many(const float* x, const float* s, int64_t n, uint8_t* out);

/* ---- block quantisers: n values -> n codes (one per byte, low nibble) + one scale byte ---- */
void orc_quant_block_nv(const float* x, int n, uint8_t* codes, uint8_t* scale);
void orc_quant_block_mx(const float* x, int n, uint8_t* codes, uint8_t* scale);
void orc_quant_block_mx8(const float* x, int n, uint8_t* codes, uint8_t* scale); /* E4M3 codes, one per byte */

/* ---- tensor quantiser (fp16 input bits). Returns ORC_OK or ORC_ERR_ARG. ---- */
int orc_quant(int role, int fmt, const uint16_t* x, int B, int H, int N, int D,
              uint8_t* codes, uint8_t* scales);

/* ---- P of one (row, tile): the two-level quantisation ----
 * x[128]: scaled scores in slot order; vis[128]: 1 if the key is visible.
 * Outputs: E[128] = exp(x - t) (0 where not visible), codes[128], scales[128/blk],
 * *t = max visible x. Returns 0 if no key is visible (outputs untouched), 1 otherwise. */
int orc_p_tile(int fmt, const float* x, const uint8_t* vis, float* E, uint8_t* codes,
               uint8_t* scales, float* t);

/* ---- quantised attention forward ----
 * rows == NULL: all B*H*N rows, out is [B,H,N,D]; else rows[r] = (b*H + h)*N + i and out is
 * [n_rows, D]. sm_scale <= 0 selects fl32(1/sqrt(D)).
 * slack (may be NULL): per output row, an upper bound on how far a correct implementation may
 * move that row (max over d) because a P rounding decision lies within its window of its
 * boundary: relative delta + 2^-20 (|x_j| + |t|) for element j of a tile with maximum t (see
 * sage_oracle.c). nthreads <= 0: OpenMP default. */
int orc_attn_fwd(int fmt, const uint8_t* q_codes, const uint8_t* q_scales,
                 const uint8_t* k_codes, const uint8_t* k_scales,
                 const uint8_t* v_codes, const uint8_t* v_scales,
                 int B, int H, int N, int D, int causal, float sm_scale,
                 const int64_t* rows, int64_t n_rows, float* out,
                 double* slack, double delta, int nthreads);

/* ---- Direct-P variant (MXFP4 operands): as orc_attn_fwd with fmt = MXFP4, except that the
 * softmax normaliser sums the dequantised P (code * block scale) instead of the unquantised
 * E (rit.work page on FP4 FlashAttention-4: the normaliser comes from the rounded values). */
int orc_attn_fwd_direct_p(const uint8_t* q_codes, const uint8_t* q_scales,
                          const uint8_t* k_codes, const uint8_t* k_scales,
                          const uint8_t* v_codes, const uint8_t* v_scales,
                          int B, int H, int N, int D, int causal, float sm_scale,
                          const int64_t* rows, int64_t n_rows, float* out,
                          double* slack, double delta, int nthreads);

/* ---- the forward with each row's log-sum-exp (plain or Direct-P): lse[r] = m + ln l, with m
 * the row's maximum scaled score and l the normaliser the output row is divided by (the sum of
 * E = exp(x - m), or with Direct-P of the dequantised P, each tile weighted by exp(t - m)).
 * lse_slack (may be NULL): per row, a bound on how far lse may move because a P rounding
 * decision lies within its window of its boundary (0 except with Direct-P). ---- */
int orc_attn_fwd_lse(int fmt, int direct_p, const uint8_t* q_codes, const uint8_t* q_scales,
                     const uint8_t* k_codes, const uint8_t* k_scales,
                     const uint8_t* v_codes, const uint8_t* v_scales,
                     int B, int H, int N, int D, int causal, float sm_scale,
                     const int64_t* rows, int64_t n_rows, float* out, double* lse,
                     double* slack, double* lse_slack, double delta, int nthreads);

/* ---- unquantised reference: softmax(c Q K^T) V in double from fp16 inputs ---- */
int orc_attn_ref_f64(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int B, int H, int N, int D, int causal, double sm_scale,
                     const int64_t* rows, int64_t n_rows, double* out, int nthreads);

/* threads OpenMP would use (1 without OpenMP) */
int orc_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
