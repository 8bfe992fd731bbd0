/*
 * sage_fp4.h — C ABI of libsage_fp4.so: microscaling-FP4 attention forward, and its 8-bit
 * backward, on AMD MI355X (gfx950).
 *
 * The operation (SageAttention3, "Microscaling FP4 Attention for Inference and An Exploration
 * of 8-Bit Training", arXiv 2505.11594; abstract, and the DeepTech article's sections on the two
 * FP4 obstacles and on FP4 inference acceleration): Q, K and V are quantised to FP4 with
 * microscaling, S = Q K^T is computed from the FP4 operands, an online softmax quantises the
 * probabilities P in two levels (each token's values scaled into [0, 448*6], then 1x16 FP4
 * microscaling), and P V is computed from FP4 operands with FP32 accumulation. Two formats:
 *   NVFP4: E2M1 codes, blocks of 16, one E4M3 scale per block (the pages' choice);
 *   MXFP4: E2M1 codes, blocks of 32, one E8M0 scale per block (the pages' comparison format).
 * A third format keeps P and V in FP8 (the rit.work page on FP4 FlashAttention-4, section on
 * what was done: its training had to leave P and V in FP8 because MXFP4 variants for them
 * diverged):
 *   MX4_PV8: Q and K as MXFP4; P and V as MXFP8, i.e. E4M3 elements in blocks of 32 with one
 *   E8M0 scale 2^(floor(log2 amax) - 8) per block; an element is the E4M3 value nearest the
 *   exact quotient x/scale, ties to even, clamped to +-448, sign bit the input's. The
 *   normaliser sums the unquantised E, as for the FP4 formats.
 *
 * Numerics (the contract the CPU oracle in oracle/ implements independently):
 *   - NVFP4 block scale: E4M3 of fl32(amax/6), round to nearest even, clamped to 448.
 *     MXFP4 block scale: 2^(floor(log2 amax) - 2), clamped to the E8M0 range; 0x00 if amax == 0.
 *   - codes: the E2M1 value nearest to the exact quotient x/scale, ties to the even code,
 *     clamped to +-6; the sign bit is the input's; a zero scale gives codes of +-0.
 *   - blocks lie along each matmul's contraction dimension: Q and K along D, V along tokens,
 *     P along keys. Inside each 128-token tile, V and P use the slot order: slot 32g + 4t + i
 *     holds token 16t + 4g + i (g < 4, t < 8, i < 4); blocks are runs of consecutive slots.
 *   - scores x = sm_scale * S; key tiles of 128 (sage_fp4_kv_tile()); per (row, tile)
 *     E = exp(x - tile max), NVFP4 P2 = 2688 E quantised per 16 slots with E4M3 scales
 *     (MXFP4: P2 = E, 32 slots, E8M0); the normaliser sums the unquantised E.
 *   - causal: key j is visible to query i iff j <= i. Exact key ties and decisions within a
 *     few ulp of a rounding boundary may round either way (exp and FP32 summation order differ
 *     from the oracle by a few ulp); codes and scales of Q, K, V are bit-exact.
 *   - exponents are formed in FP32 relative to the tile maximum, carried with its exact
 *     rounding error, so the outputs stay within the same bar at any score magnitude.
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers owned by the caller; the library allocates
 *     nothing, keeps no state and is thread-safe. Inputs are read-only.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously;
 *     nothing synchronises.
 *   - arguments are validated on the host before anything is enqueued; a negative sage_status
 *     is returned on error and nothing is launched. SAGE_ERR_HIP reports a launch failure
 *     (hipGetLastError after the launch).
 *   - every pointer must be 16-byte aligned; tensors are dense and row-major.
 *   - supported: D in {64, 128}; 1 <= N <= 1048576; B*H <= 65535; B*H*N*D < 2^36 (a launch
 *     grid limit, larger than three fp16 tensors that fit in HBM). N_q == N_k, no GQA.
 */
#ifndef SAGE_FP4_H
#define SAGE_FP4_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SAGE_FMT_NVFP4 = 0, SAGE_FMT_MXFP4 = 1, SAGE_FMT_MX4_PV8 = 2 } sage_fmt_t;
typedef enum { SAGE_ROLE_Q = 0, SAGE_ROLE_K = 1, SAGE_ROLE_V = 2 } sage_role_t;
typedef enum { SAGE_OUT_F16 = 0, SAGE_OUT_F32 = 1 } sage_out_t;
typedef enum { SAGE_BWD_PREP = 0, SAGE_BWD_DKDV = 1, SAGE_BWD_DQ = 2 } sage_bwd_stage_t;
typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_NULL = -1,     /* a required pointer is NULL */
  SAGE_ERR_SHAPE = -2,    /* B, H or N out of range */
  SAGE_ERR_HEAD_DIM = -3, /* D not in {64, 128} */
  SAGE_ERR_ALIGN = -4,    /* a pointer is not 16-byte aligned */
  SAGE_ERR_ENUM = -5,     /* bad format, role or output type */
  SAGE_ERR_HIP = -6,      /* the HIP runtime reported an error for the launch */
  SAGE_ERR_WORKSPACE = -7 /* the workspace is smaller than the call needs */
} sage_status_t;

/* Library version (major*10000 + minor*100 + patch). */
int sage_fp4_version(void);

/* Key-tile size of the online softmax (128). The per-(row, tile) first level of P makes the
 * result depend on it. */
int sage_fp4_kv_tile(void);

/* Token held by `slot` (0..127) of a 128-token tile in the slot order above; -1 if out of range. */
int sage_fp4_slot_token(int slot);

/* Bytes needed for the codes / scales of one quantised tensor (0 for invalid arguments).
 *   Q, K: codes [B,H,N,D/2], scales [B,H,N,D/16] (NVFP4) or [B,H,N,D/32] (MXFP4);
 *   V:    codes [B,H,Np/128,D,64], scales [B,H,Np/128,D,8] or [B,H,Np/128,D,4],
 *         Np = ceil(N/128)*128; MX4_PV8: codes [B,H,Np/128,D,128] (one E4M3 byte per element),
 *         scales [B,H,Np/128,D,4]. Tile by tile: one 128-token tile's codes, and its scales,
 *         for every channel are one contiguous run (the quantiser writes, and the attention
 *         reads, whole runs); inside a tile a channel's 128 slots are in slot order. */
size_t sage_fp4_codes_bytes(int role, int fmt, int B, int H, int N, int D);
size_t sage_fp4_scales_bytes(int role, int fmt, int B, int H, int N, int D);

/* Quantise one fp16 tensor x [B,H,N,D] (dense, row-major) for its role in the attention.
 * Q and K: blocks of 16 (32) consecutive channels of each token; codes [B,H,N,D/2] with
 * element 2i in the low nibble of byte i; scales one byte per block.
 * V: blocks along tokens. codes [B,H,Np/128,D,64] hold, for each 128-token tile and channel d,
 * the tile's tokens in slot order (two per byte, low nibble first; MX4_PV8: [B,H,Np/128,D,128],
 * one byte each); token positions >= N hold 0. scales [B,H,Np/128,D,128/blk], one per block
 * of consecutive slots. With MX4_PV8, Q and K are quantised exactly as with MXFP4.
 * One kernel launch. Inputs must be finite. */
int sage_fp4_quant(int role, int fmt, const void* x, int B, int H, int N, int D,
                   void* codes, void* scales, void* stream);

/* Attention forward from quantised operands (as produced by sage_fp4_quant with the same fmt).
 * out [B,H,N,D], fp16 (SAGE_OUT_F16) or fp32 (SAGE_OUT_F32), dense row-major.
 * sm_scale <= 0 selects fl32(1/sqrt(D)). causal != 0 applies the top-left causal mask.
 * One kernel launch. */
int sage_fp4_attn_fwd(int fmt, const void* q_codes, const void* q_scales,
                      const void* k_codes, const void* k_scales,
                      const void* v_codes, const void* v_scales,
                      int B, int H, int N, int D, int causal, float sm_scale,
                      void* out, int out_dtype, void* stream);

/* Direct-P variant of the MXFP4 attention forward (the rit.work page on FP4 FlashAttention-4,
 * section on what was done): the scores go straight to the MXFP4 codes of P consumed by the
 * second matmul, and the softmax normaliser is the sum of those rounded values (the decoded
 * E2M1 codes times their E8M0 block scales) instead of the unquantised E. Everything else -
 * operands (MXFP4 codes and scales from sage_fp4_quant with SAGE_FMT_MXFP4), tiles, P
 * quantisation, masking, output layout, validation and errors - is that of sage_fp4_attn_fwd
 * with fmt = SAGE_FMT_MXFP4. One kernel launch. */
int sage_fp4_attn_fwd_direct_p(const void* q_codes, const void* q_scales,
                               const void* k_codes, const void* k_scales,
                               const void* v_codes, const void* v_scales,
                               int B, int H, int N, int D, int causal, float sm_scale,
                               void* out, int out_dtype, void* stream);

/* Attention forward that also returns each row's softmax normaliser as a log-sum-exp: the
 * statistic of the online softmax the pages fuse with the P quantisation (DeepTech article,
 * section on FP4 inference and its hardware implementation), kept for a backward pass of the
 * pages' 8-bit training attention (abstract, second contribution) and for merging partial
 * results. Same operands, output, validation and errors as sage_fp4_attn_fwd (direct_p == 0) or
 * sage_fp4_attn_fwd_direct_p (direct_p != 0, which needs fmt = SAGE_FMT_MXFP4, else
 * SAGE_ERR_ENUM), plus:
 *   lse  device pointer, fp32 [B,H,N], 16-byte aligned, caller-owned; NULL is SAGE_ERR_NULL.
 *        lse[b,h,i] = ln sum_j exp(x_ij) over the keys j visible to query i, x = sm_scale * S
 *        with S from the quantised Q and K, i.e. the normaliser the output row was divided by;
 *        with direct_p, ln sum over tiles of exp(t) * (sum of the tile's dequantised P values),
 *        t the tile's row maximum of x.
 * For key ranges that are unions of whole 128-key tiles, results computed separately over each
 * range r merge exactly (up to FP32 rounding) as out = sum_r exp(lse_r - lse) out_r with
 * lse = ln sum_r exp(lse_r), because P is quantised per tile. One kernel launch. */
int sage_fp4_attn_fwd_lse(int fmt, int direct_p, const void* q_codes, const void* q_scales,
                          const void* k_codes, const void* k_scales,
                          const void* v_codes, const void* v_scales,
                          int B, int H, int N, int D, int causal, float sm_scale,
                          void* out, int out_dtype, float* lse, void* stream);

/* Bytes of the buffer sage_fp4_kv16_prep fills (0 for invalid arguments): 4*B*H*Np*D,
 * Np = ceil(N/128)*128. */
size_t sage_fp4_kv16_bytes(int B, int H, int N, int D);

/* NVFP4 K and V dequantised once, exactly, to fp16 (the DeepTech article, section on FP4
 * inference and its hardware implementation, for the operands; every value is a code times its
 * E4M3 block scale, at most 6 significant bits in 2^-10 .. 2688, so fp16 holds it exactly).
 * The attention kernel otherwise dequantises each K and V tile in every query tile that reads
 * it; sage_fp4_attn_fwd_kv16 reads this buffer instead, and one buffer serves any number of
 * attention calls over the same K and V.
 *   k_codes, k_scales, v_codes, v_scales   NVFP4, as from sage_fp4_quant(SAGE_FMT_NVFP4).
 *   kv16   device buffer of at least sage_fp4_kv16_bytes(B,H,N,D) bytes, caller-owned; it
 *          receives K-hat fp16 [B,H,Np,D] (rows >= N zero) followed by V-hat fp16
 *          [B,H,Np/128,D,128] (the V codes' tile-major slot order; positions >= N zero).
 *          A smaller kv16_bytes is SAGE_ERR_WORKSPACE.
 * Validation and errors as for sage_fp4_quant. One kernel launch. */
int sage_fp4_kv16_prep(const void* k_codes, const void* k_scales,
                       const void* v_codes, const void* v_scales,
                       int B, int H, int N, int D, void* kv16, size_t kv16_bytes, void* stream);

/* NVFP4 quantisation of K or V that also fills that operand's part of the kv16 buffer, in the
 * same pass over x (the DeepTech article, section on FP4 inference and its hardware
 * implementation, for the operands): codes and scales are those sage_fp4_quant(role,
 * SAGE_FMT_NVFP4, ...) writes, and the kv16 bytes those sage_fp4_kv16_prep writes from them, bit
 * for bit. role SAGE_ROLE_K writes K-hat (the first half of kv16), SAGE_ROLE_V writes V-hat (the
 * second half); the other half is left as it is, so one call per role fills the buffer.
 *   role    SAGE_ROLE_K or SAGE_ROLE_V, else SAGE_ERR_ENUM.
 *   kv16    device buffer of at least sage_fp4_kv16_bytes(B,H,N,D) bytes, caller-owned, 16-byte
 *           aligned; a smaller kv16_bytes is SAGE_ERR_WORKSPACE.
 * x, codes, scales, the shape, validation and errors as for sage_fp4_quant. Nothing is written
 * when an error is returned before the launch. One kernel launch. */
int sage_fp4_quant_kv16(int role, const void* x, int B, int H, int N, int D,
                        void* codes, void* scales, void* kv16, size_t kv16_bytes, void* stream);

/* NVFP4 attention forward with K and V from sage_fp4_kv16_prep's buffer: the same operation,
 * tiles and arithmetic as sage_fp4_attn_fwd(SAGE_FMT_NVFP4, ...) on the codes kv16 was made from,
 * and the same output bit for bit (and lse as sage_fp4_attn_fwd_lse). It reads 2 bytes per K and
 * V element instead of 0.56, so it pays where the dequantisation it saves outweighs that:
 * long sequences, or one kv16 buffer reused by several calls.
 *   q_codes, q_scales   NVFP4, as from sage_fp4_quant(SAGE_ROLE_Q, SAGE_FMT_NVFP4).
 *   kv16                the buffer, kv16_bytes >= sage_fp4_kv16_bytes(B,H,N,D), else
 *                       SAGE_ERR_WORKSPACE.
 *   lse                 NULL, or fp32 [B,H,N] (16-byte aligned) receiving each row's
 *                       log-sum-exp as in sage_fp4_attn_fwd_lse.
 * Other arguments, validation and errors as for sage_fp4_attn_fwd. One kernel launch. */
int sage_fp4_attn_fwd_kv16(const void* q_codes, const void* q_scales,
                           const void* kv16, size_t kv16_bytes,
                           int B, int H, int N, int D, int causal, float sm_scale,
                           void* out, int out_dtype, float* lse, void* stream);

/* Bytes of device workspace sage_fp4_attn_bwd needs for this shape (0 for invalid arguments).
 * About 4*B*H*N*D + 3*B*H*D*Np64 bytes, Np64 = ceil(N/64)*64. */
size_t sage_fp4_attn_bwd_workspace_bytes(int B, int H, int N, int D);

/* 8-bit attention backward (SageAttention3's SageBwd: DeepTech article, sections on the third
 * difficulty and on INT8 attention for training; the rit.work page on FP4 FlashAttention-4,
 * section on what was done, for the forward handing the backward its quantised Q and K, their
 * scales and the normaliser). Gradients of the attention whose forward is sage_fp4_attn_fwd_lse,
 * with c = sm_scale (<= 0 selects fl32(1/sqrt(D))) and the same causal mask:
 *   S = Q^ K^T from the FP4 codes (exact), P = exp(c S - lse), dP = dO V^T (16-bit operands,
 *   fp32 accumulation), D_i = sum_d dO_id O_id, dS = P (dP - D),
 *   dV = P^T dO, dK = c dS^T Q^, dQ = c dS K^ on INT8 operands. Each INT8 operand carries one
 *   fp32 scale per row (the index not contracted) and per block of 64 contraction indices:
 *   P^T and dS^T per (key, 64-query block), dS per (query, 64-key block), dO, Q^ and K^ per
 *   (channel, 64-token block); the 64 values x of a block with a = max|x| get the scale
 *   fl32(a/127) and codes rne(fl32(x * fl32(127/a))) in [-127, 127]. Codes that lie within a
 *   few ulp of a rounding boundary may round either way (fp32 summation order).
 * Arguments:
 *   fmt                  format of the forward's Q and K codes (NVFP4; MXFP4 and MX4_PV8 both
 *                        have MXFP4 Q and K); codes and scales as from sage_fp4_quant.
 *   v, o, dout           fp16 [B,H,N,D]: V, the forward's output and the output gradient.
 *   lse                  fp32 [B,H,N] from sage_fp4_attn_fwd_lse.
 *   dq, dk, dv           [B,H,N,D] outputs, fp16 or fp32 per out_dtype, fully written.
 *   workspace            device memory of at least sage_fp4_attn_bwd_workspace_bytes(B,H,N,D)
 *                        bytes (workspace_bytes), 16-byte aligned, caller-owned; its contents
 *                        on entry are ignored, and on return it holds, at 256-byte aligned
 *                        offsets in this order: Q^ and K^ as bf16 [B,H,N,D] (with MXFP4 Q and
 *                        K, these two regions begin instead with their E8M0 scales as
 *                        [B,H,Np64/64,D/32,16,4] bytes, byte [b][g][c][s] belonging to token
 *                        min(64b + 16s + c, N - 1), block g); the INT8 codes of
 *                        Q^, K^ and dO, each [B,H,D,Np64] with the tokens of every 64-token
 *                        block in slot order (slot 16g + 4s + i holds token 16s + 4g + i, zero
 *                        past N); their scales, fp32 [B,H,Np64/64,D] each; D and lse*log2(e),
 *                        fp32 [B,H,Np64] each (past N: 0 and 1e30).
 *                        Calls that share a workspace must not overlap.
 * Errors as for the forward; a workspace below the needed size is SAGE_ERR_WORKSPACE. Five
 * kernel launches on `stream` (three operand preparations, dK/dV, dQ); no atomics, so results
 * are deterministic. */
int sage_fp4_attn_bwd(int fmt, const void* q_codes, const void* q_scales,
                      const void* k_codes, const void* k_scales,
                      const void* v, const void* o, const void* dout, const float* lse,
                      int B, int H, int N, int D, int causal, float sm_scale,
                      void* dq, void* dk, void* dv, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* One stage of sage_fp4_attn_bwd, for callers that time or schedule the stages separately: the
 * full call is exactly SAGE_BWD_PREP, SAGE_BWD_DKDV, SAGE_BWD_DQ in that order on one stream
 * with one workspace. Same arguments, validation and errors (a bad `stage` is SAGE_ERR_ENUM).
 *   SAGE_BWD_PREP  three launches: fills the workspace from the Q/K codes, dout and o.
 *   SAGE_BWD_DKDV  one launch: writes dk and dv from the workspace, v, dout and lse.
 *   SAGE_BWD_DQ    one launch: writes dq from the workspace, v, dout and lse.
 * A gradient stage reads a workspace filled by a preparation stage of the same arguments;
 * pointers a stage does not use are still validated. */
int sage_fp4_attn_bwd_stage(int stage, int fmt, const void* q_codes, const void* q_scales,
                            const void* k_codes, const void* k_scales,
                            const void* v, const void* o, const void* dout, const float* lse,
                            int B, int H, int N, int D, int causal, float sm_scale,
                            void* dq, void* dk, void* dv, int out_dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device-resident workspace of sage_fp4_attn_bwd_noalloc: 64 MiB, enough for
 * shapes with about B*H*N*D <= 8M elements (e.g. B=1, H=16, N=4096, D=128). */
#define SAGE_BWD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* sage_fp4_attn_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc. Same arguments,
 * computation, validation and results (bit for bit) as sage_fp4_attn_bwd, without `workspace`
 * and `workspace_bytes`: the workspace is an array of SAGE_BWD_NOALLOC_SCRATCH_BYTES inside the
 * library, one copy per GPU (the GPU of `stream`; the current one for the null stream), held
 * until the process ends. The first call on a GPU looks up that copy's address
 * (hipGetSymbolAddress); no call allocates, frees or clears memory. Shapes whose workspace
 * (sage_fp4_attn_bwd_workspace_bytes) exceeds the array return SAGE_ERR_WORKSPACE before any
 * launch. Every call on one GPU uses the same array and leaves its contents behind (the next
 * call overwrites what it reads before reading it), so calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller. */
int sage_fp4_attn_bwd_noalloc(int fmt, const void* q_codes, const void* q_scales,
                              const void* k_codes, const void* k_scales,
                              const void* v, const void* o, const void* dout, const float* lse,
                              int B, int H, int N, int D, int causal, float sm_scale,
                              void* dq, void* dk, void* dv, int out_dtype, void* stream);

/* Static description of a status code. */
const char* sage_fp4_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_FP4_H */
