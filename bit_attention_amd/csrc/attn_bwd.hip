// attn_bwd.hip — the 8-bit attention backward for gfx950.
//
// SageAttention3 (arXiv 2505.11594), DeepTech article, sections on the third difficulty and on
// INT8 attention for training: six of the seven matmuls of attention training run in INT8, and
// the one the gradient of the attention map comes from stays in 16 bits. The rit.work page on
// FP4 FlashAttention-4 ("What was done"): the forward hands the backward its quantised Q and K,
// their scales and the normaliser. With c the softmax scale and lse the forward's row
// log-sum-exp:
//   S = Q^ K^T (exact, from the FP4 codes)   P = exp(c S - lse)   dP = dO V^T (fp16 operands)
//   D_i = sum_d dO_id O_id   dS = P (dP - D)   dV = P^T dO   dK = c dS^T Q^   dQ = c dS K^
// with the last three on INT8 operands, each carrying one fp32 scale per row (the index that is
// not contracted) and per 64-wide block of the contraction: P^T and dS^T per (key, 64-query
// block), dS per (query, 64-key block), dO, Q^ and K^ per (channel, 64-token block). The 64
// values x of one block, with a = max|x|, get the scale fl32(a / 127) and the codes
// rne(fl32(x * fl32(127 / a))).
//
// CDNA4 design.
//   - prep kernels, one workgroup per (batch*head, 64-token block): Q^ and K^ are dequantised
//     from FP4 to bf16 (exact: a code times its scale has at most 6 significant bits and lies
//     in bf16's exponent range), and Q^, K^ and dO are encoded to INT8 per (channel, block),
//     stored channel-major in the token order below; the dO prep also forms D_i in fp32.
//   - dK/dV kernel, one workgroup of 4 waves per (batch*head, 64-key block): each wave owns 16
//     keys and keeps their K^ (bf16) and V (fp16) rows as MFMA B operands in registers while the
//     workgroup stages 64-query tiles through LDS. S = Q^ K^T and dP = dO V^T take 16x16x32
//     MFMAs; a lane then holds 16 (query, key) values of one key, at queries 16s + 4g + i
//     (subtile s, lane group g, element i). P and dS are therefore lane-local, a key's block
//     maximum takes two cross-lane swaps, and a lane's 16 codes are directly the A operand of a
//     16x16x64 INT8 MFMA whose K slots 16g + 4s + i hold those queries; the INT8 dO and Q^ are
//     stored in that slot order. Two workgroups fit on a CU (57 KB of LDS each at D = 128).
//   - dQ kernel: the mirror image, one wave per 16 queries looping over 64-key tiles. dQ gets
//     a kernel of its own instead of atomic adds, so every result is deterministic.
#include <type_traits>

#include "device.h"

namespace sage {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 f16;

constexpr int BB = 64;                          // token block of the INT8 operands and tile size
constexpr float LOG2E = 1.4426950408889634f;

// Token held by slot p of a 64-token block: slot 16g + 4s + i holds token 16s + 4g + i (an
// involution). A wave's 16x16 MFMA results for four 16-token subtiles put token 16s + 4g + i in
// lane group g, subtile s, element i; the 16x16x64 INT8 MFMA reads K slots 16g + [0, 16) from
// lane group g.
__host__ __device__ inline int slot_token64(int p) { return 16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3); }

// fl32(a / b) and fl32(b / a) for the INT8 scale: double division rounded once more to fp32
// equals the correctly rounded fp32 quotient (53 >= 2 * 24 + 2).
__device__ __forceinline__ float div_rn(float a, float b) { return (float)((double)a / (double)b); }

// Four integers in [-127, 127] -> one dword, the first in the low byte.
__device__ __forceinline__ int pack4(int a, int b, int c, int d) {
  return (a & 0xFF) | ((b & 0xFF) << 8) | ((c & 0xFF) << 16) | ((d & 0xFF) << 24);
}

// ---------------------------------------------------------------------------------------------
// Prep: one workgroup per (block of 64 tokens, batch*head). SRC 0: NVFP4 codes, 1: MXFP4 codes
// (both also write the bf16 values), 2: fp16 dO (also writes D_i from dO and O).
// ---------------------------------------------------------------------------------------------
template <int D, int SRC>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const f16* __restrict__ x, const f16* __restrict__ o,
                                                       int N, int Np, __bf16* __restrict__ xh,
                                                       int8_t* __restrict__ q8, float* __restrict__ q8s,
                                                       float* __restrict__ dl) {
  constexpr int VPT = D / 4;      // values per thread in the row phase (64 rows x D / 256)
  constexpr int TPR = D / VPT;    // threads per token row (4)
  constexpr int TPC = 256 / D;    // threads per channel in the channel phase
  constexpr int PP = BB / TPC;    // slots per thread in the channel phase
  __shared__ float sx[BB][D + 1];
  const int blk = blockIdx.x, nb = Np / BB;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;

  // row phase: token n, channels [ch * VPT, (ch + 1) * VPT)
  {
    const int n = tid / TPR, ch = tid % TPR;
    const int tok = blk * BB + n;
    float v[VPT];
    if (tok < N) {
      const int64_t row = bh * N + tok;
      if constexpr (SRC == 2) {
        const v8h* xp = reinterpret_cast<const v8h*>(x + row * D + ch * VPT);
        const v8h* op = reinterpret_cast<const v8h*>(o + row * D + ch * VPT);
        float dot = 0.0f;
#pragma unroll
        for (int u = 0; u < VPT / 8; ++u) {
          const v8h a = xp[u], b = op[u];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[8 * u + e] = (float)a[e];
            dot = __builtin_fmaf((float)a[e], (float)b[e], dot);
          }
        }
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        if (ch == 0) dl[row] = dot;
      } else {
        constexpr int blkv = SRC == 0 ? 16 : 32;
        const unsigned* cw = reinterpret_cast<const unsigned*>(codes + row * (D / 2) + ch * (VPT / 2));
        const uint8_t* sc = scales + row * (D / blkv);
#pragma unroll
        for (int u = 0; u < VPT / 8; ++u) {
          const unsigned wv = cw[u];
          const unsigned sb = sc[(ch * VPT + 8 * u) / blkv];
          float s;
          if constexpr (SRC == 0) s = e4m3_decode(sb);
          else s = sb == 0 ? as_f(0x00400000u) : sb == 255 ? as_f(0x7FC00000u) : as_f(sb << 23);
          const v2h h[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 3)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * u + 2 * e] = (float)h[e][0] * s;
            v[8 * u + 2 * e + 1] = (float)h[e][1] * s;
          }
        }
        __bf16* dst = xh + row * D + ch * VPT;
#pragma unroll
        for (int u = 0; u < VPT / 8; ++u) {
          v8bf b;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)v[8 * u + e];
          *reinterpret_cast<v8bf*>(dst + 8 * u) = b;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < VPT; ++u) v[u] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) sx[n][ch * VPT + u] = v[u];
  }
  __syncthreads();

  // channel phase: channel d, slots [h * PP, (h + 1) * PP)
  {
    const int d = tid / TPC, h = tid % TPC;
    float a = 0.0f;
#pragma unroll
    for (int p = 0; p < PP; ++p) a = fmaxf(a, fabsf(sx[slot_token64(h * PP + p)][d]));
    a = fmaxf(a, __shfl_xor(a, 1));
    if constexpr (TPC == 4) a = fmaxf(a, __shfl_xor(a, 2));
    const float r = a > 0.0f ? div_rn(127.0f, a) : 0.0f;
    int cq[PP];
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const float t = __builtin_rintf(sx[slot_token64(h * PP + p)][d] * r);
      cq[p] = (int)fminf(fmaxf(t, -127.0f), 127.0f);
    }
    int8_t* dst = q8 + (bh * D + d) * Np + blk * BB + h * PP;
#pragma unroll
    for (int u = 0; u < PP / 16; ++u) {
      v4i wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[e] = pack4(cq[16 * u + 4 * e], cq[16 * u + 4 * e + 1], cq[16 * u + 4 * e + 2], cq[16 * u + 4 * e + 3]);
      *reinterpret_cast<v4i*>(dst + 16 * u) = wv;
    }
    if (h == 0) q8s[(bh * D + d) * nb + blk] = a > 0.0f ? div_rn(a, 127.0f) : 0.0f;
  }
}

// ---------------------------------------------------------------------------------------------
// Shared pieces of the two gradient kernels.
// ---------------------------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int RP = D + 8;        // LDS row pitch (elements) of the 16-bit tiles
  static constexpr int CP = BB + 16;      // LDS row pitch (bytes) of the INT8 tiles
  static constexpr int KK = D / 32;       // k steps of the 16x16x32 MFMAs
  static constexpr int NN = D / 16;       // 16-channel output subtiles
};

// Stage one 64-token tile: rows [t0, t0 + 64) of a bf16 and an fp16 [.., N, D] tensor (zero past
// N), the INT8 codes [D][64] of the block and its per-channel scales.
template <int D>
__device__ __forceinline__ void stage_tile(int tid, int64_t bh, int N, int Np, int t0, int blk,
                                           const __bf16* __restrict__ a16, const f16* __restrict__ b16,
                                           const int8_t* __restrict__ c8, const float* __restrict__ c8s,
                                           __bf16* sA, f16* sB, int8_t* sC, float* sCs) {
  using T = BwdTile<D>;
#pragma unroll
  for (int u = 0; u < BB * D / 8 / 256; ++u) {
    const int idx = tid + 256 * u, row = idx / (D / 8), ch = idx % (D / 8);
    const int tok = t0 + row;
    v4u va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
    if (tok < N) {
      va = *reinterpret_cast<const v4u*>(a16 + (bh * N + tok) * D + 8 * ch);
      vb = *reinterpret_cast<const v4u*>(b16 + (bh * N + tok) * D + 8 * ch);
    }
    *reinterpret_cast<v4u*>(sA + row * T::RP + 8 * ch) = va;
    *reinterpret_cast<v4u*>(sB + row * T::RP + 8 * ch) = vb;
  }
#pragma unroll
  for (int u = 0; u < (D * 4 + 255) / 256; ++u) {
    const int idx = tid + 256 * u;
    if (idx < D * 4) {
      const int d = idx >> 2, ch = idx & 3;
      *reinterpret_cast<v4u*>(sC + d * T::CP + 16 * ch) =
          *reinterpret_cast<const v4u*>(c8 + (bh * D + d) * Np + t0 + 16 * ch);
    }
  }
  if (tid < D) sCs[tid] = c8s[(bh * D + tid) * (Np / BB) + blk];
}

// Codes of 16 values held by a lane (four subtiles s of four elements i) with a common
// reciprocal scale r; byte 4s + i of the result is the code of value [s][i]. One fma adds
// 1.5 * 2^23 to the exact product x * r, which rounds it to the nearest integer (ties to even)
// in the low mantissa bits; the low byte of the result's bits is the two's complement byte of
// that integer. This is rne(fl32(x * r)) except when x * r lies within half an fp32 ulp of a
// half-integer, where either rounding is within the contract. |x| <= the block maximum a and
// r = fl32(127 / a) keep |x * r| below 127.5, so the code lies in [-127, 127] without a clamp.
// v_perm_b32 gathers four bytes into one dword.
__device__ __forceinline__ v4i codes16(const float (&x)[4][4], float r) {
  constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
  v4i out;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = as_u(__builtin_fmaf(x[s][i], r, MAGIC));
    const unsigned lo = __builtin_amdgcn_perm(w[1], w[0], 0x0C0C0400u);  // bytes w0.b0, w1.b0, 0, 0
    const unsigned hi = __builtin_amdgcn_perm(w[3], w[2], 0x04000C0Cu);  // bytes 0, 0, w2.b0, w3.b0
    out[s] = (int)(lo | hi);
  }
  return out;
}

template <bool OUT_F32>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (OUT_F32) reinterpret_cast<float*>(out)[idx] = v;
  else reinterpret_cast<f16*>(out)[idx] = (f16)v;
}

// ---------------------------------------------------------------------------------------------
// dK and dV: one workgroup per (batch*head, 64-key block).
// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const __bf16* __restrict__ qh, const __bf16* __restrict__ kh, const f16* __restrict__ v,
    const f16* __restrict__ dout, const int8_t* __restrict__ q8, const float* __restrict__ q8s,
    const int8_t* __restrict__ do8, const float* __restrict__ do8s, const float* __restrict__ lse,
    const float* __restrict__ dl, int N, int Np, int BH, float c, void* __restrict__ dk, void* __restrict__ dv) {
  using T = BwdTile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[BB * T::RP];
  __shared__ __attribute__((aligned(16))) f16 sdO[BB * T::RP];
  __shared__ __attribute__((aligned(16))) int8_t sQ8[D * T::CP];
  __shared__ __attribute__((aligned(16))) int8_t sdO8[D * T::CP];
  __shared__ float sQs[D], sdOs[D];
  __shared__ __attribute__((aligned(16))) float sL[BB], sD[BB];

  const int nb = Np / BB;
  const int w = xcd_work(blockIdx.x, BH * nb);
  const int64_t bh = w / nb;
  const int kb = w % nb;  // causal: the heaviest key blocks (most query tiles) of a head first
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, g = l >> 4, col = l & 15;
  const int key = kb * BB + wave * 16 + col;

  v8bf kreg[T::KK];
  v8h vreg[T::KK];
#pragma unroll
  for (int kk = 0; kk < T::KK; ++kk) {
    if (key < N) {
      kreg[kk] = *reinterpret_cast<const v8bf*>(kh + (bh * N + key) * D + 32 * kk + 8 * g);
      vreg[kk] = *reinterpret_cast<const v8h*>(v + (bh * N + key) * D + 32 * kk + 8 * g);
    } else {
      kreg[kk] = v8bf{};
      vreg[kk] = v8h{};
    }
  }
  v4f accK[T::NN], accV[T::NN];
#pragma unroll
  for (int n = 0; n < T::NN; ++n) accK[n] = accV[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const float cl2e = c * LOG2E;

  // non-causal: each workgroup starts at its own query tile (kb) and wraps around, so the
  // workgroups of a head do not all read the same tile at the same time
  const int it0 = CAUSAL ? kb : 0, nit = CAUSAL ? nb - kb : nb;
  for (int it = 0; it < nit; ++it) {
    const int qt = CAUSAL ? it0 + it : (kb + it) % nb;
    const int q0 = qt * BB;
    __syncthreads();
    stage_tile<D>(tid, bh, N, Np, q0, qt, qh, dout, q8, q8s, sQ, sdO, sQ8, sQs);
    if (tid >= 128 && tid < 128 + D) sdOs[tid - 128] = do8s[(bh * D + tid - 128) * nb + qt];
    if (tid < BB) sL[tid] = q0 + tid < N ? lse[bh * N + q0 + tid] * LOG2E : 0.0f;
    else if (tid < 2 * BB) sD[tid - BB] = q0 + tid - BB < N ? dl[bh * N + q0 + tid - BB] : 0.0f;
#pragma unroll
    for (int u = 0; u < (D * 4 + 255) / 256; ++u) {
      const int idx = tid + 256 * u;
      if (idx < D * 4) {
        const int d = idx >> 2, ch = idx & 3;
        *reinterpret_cast<v4u*>(sdO8 + d * T::CP + 16 * ch) =
            *reinterpret_cast<const v4u*>(do8 + (bh * D + d) * Np + q0 + 16 * ch);
      }
    }
    __syncthreads();

    auto tile = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      float P[4][4], dS[4][4];
      float pmax = 0.0f, smax = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v4f sc = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
          const v8bf a = *reinterpret_cast<const v8bf*>(sQ + (16 * s + col) * T::RP + 32 * kk + 8 * g);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kreg[kk], sc, 0, 0, 0);
          const v8h b = *reinterpret_cast<const v8h*>(sdO + (16 * s + col) * T::RP + 32 * kk + 8 * g);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, vreg[kk], dp, 0, 0, 0);
        }
        const v4f L4 = *reinterpret_cast<const v4f*>(sL + 16 * s + 4 * g);
        const v4f D4 = *reinterpret_cast<const v4f*>(sD + 16 * s + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = q0 + 16 * s + 4 * g + i;
          const bool ok = FULL || (qi < N && key < N && (!CAUSAL || key <= qi));
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cl2e, -L4[i]));
          const float p = ok ? e : 0.0f;
          P[s][i] = p;
          dS[s][i] = p * (dp[i] - D4[i]);
          pmax = fmaxf(pmax, p);
          smax = fmaxf(smax, fabsf(dS[s][i]));
        }
      }
      pmax = xg_max(pmax);
      smax = xg_max(smax);
      const v4i aP = codes16(P, pmax > 0.0f ? div_rn(127.0f, pmax) : 0.0f);
      const v4i aS = codes16(dS, smax > 0.0f ? div_rn(127.0f, smax) : 0.0f);
      const float sP = pmax > 0.0f ? div_rn(pmax, 127.0f) : 0.0f;
      const float sS = smax > 0.0f ? div_rn(smax, 127.0f) : 0.0f;
      // the accumulator rows are keys 16 * wave + 4g + i; lane 4g + i holds their scales
      float rP[4], rS[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rP[i] = __shfl(sP, 4 * g + i);
        rS[i] = __shfl(sS, 4 * g + i);
      }
#pragma unroll
      for (int n = 0; n < T::NN; ++n) {
        const v4i bo = *reinterpret_cast<const v4i*>(sdO8 + (16 * n + col) * T::CP + 16 * g);
        const v4i bq = *reinterpret_cast<const v4i*>(sQ8 + (16 * n + col) * T::CP + 16 * g);
        const v4i rv = __builtin_amdgcn_mfma_i32_16x16x64_i8(aP, bo, v4i{0, 0, 0, 0}, 0, 0, 0);
        const v4i rk = __builtin_amdgcn_mfma_i32_16x16x64_i8(aS, bq, v4i{0, 0, 0, 0}, 0, 0, 0);
        const float co = sdOs[16 * n + col], cq = sQs[16 * n + col];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accV[n][i] = __builtin_fmaf((float)rv[i], rP[i] * co, accV[n][i]);
          accK[n][i] = __builtin_fmaf((float)rk[i], rS[i] * cq, accK[n][i]);
        }
      }
    };
    // one variant with the per-element mask: a second, mask-free one for interior tiles
    // raises the register count past 256
    tile(std::false_type{});
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = kb * BB + wave * 16 + 4 * g + i;
    if (kr >= N) continue;
#pragma unroll
    for (int n = 0; n < T::NN; ++n) {
      const int64_t idx = (bh * N + kr) * D + 16 * n + col;
      store_out<OUT_F32>(dk, idx, c * accK[n][i]);
      store_out<OUT_F32>(dv, idx, accV[n][i]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ: one workgroup per (batch*head, 64-query block).
// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ qh, const __bf16* __restrict__ kh, const f16* __restrict__ v,
    const f16* __restrict__ dout, const int8_t* __restrict__ k8, const float* __restrict__ k8s,
    const float* __restrict__ lse, const float* __restrict__ dl, int N, int Np, int BH, float c,
    void* __restrict__ dq) {
  using T = BwdTile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[BB * T::RP];
  __shared__ __attribute__((aligned(16))) f16 sV[BB * T::RP];
  __shared__ __attribute__((aligned(16))) int8_t sK8[D * T::CP];
  __shared__ float sKs[D];

  const int nb = Np / BB;
  const int w = xcd_work(blockIdx.x, BH * nb);
  const int64_t bh = w / nb;
  const int qb = CAUSAL ? nb - 1 - w % nb : w % nb;  // causal: the heaviest query blocks first
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, g = l >> 4, col = l & 15;
  const int query = qb * BB + wave * 16 + col;

  v8bf qreg[T::KK];
  v8h oreg[T::KK];
  float Lq = 0.0f, Dq = 0.0f;
#pragma unroll
  for (int kk = 0; kk < T::KK; ++kk) {
    if (query < N) {
      qreg[kk] = *reinterpret_cast<const v8bf*>(qh + (bh * N + query) * D + 32 * kk + 8 * g);
      oreg[kk] = *reinterpret_cast<const v8h*>(dout + (bh * N + query) * D + 32 * kk + 8 * g);
    } else {
      qreg[kk] = v8bf{};
      oreg[kk] = v8h{};
    }
  }
  if (query < N) {
    Lq = lse[bh * N + query] * LOG2E;
    Dq = dl[bh * N + query];
  }
  v4f acc[T::NN];
#pragma unroll
  for (int n = 0; n < T::NN; ++n) acc[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const float cl2e = c * LOG2E;

  // non-causal: each workgroup starts at its own key tile (qb) and wraps around
  const int nit = CAUSAL ? qb + 1 : nb;
  for (int it = 0; it < nit; ++it) {
    const int kt = CAUSAL ? it : (qb + it) % nb;
    const int k0 = kt * BB;
    __syncthreads();
    stage_tile<D>(tid, bh, N, Np, k0, kt, kh, v, k8, k8s, sK, sV, sK8, sKs);
    __syncthreads();

    const bool full = k0 + BB <= N && qb * BB + BB <= N && (!CAUSAL || kt < qb);
    auto tile = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      float dS[4][4];
      float smax = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v4f sc = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
          const v8bf a = *reinterpret_cast<const v8bf*>(sK + (16 * s + col) * T::RP + 32 * kk + 8 * g);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[kk], sc, 0, 0, 0);
          const v8h b = *reinterpret_cast<const v8h*>(sV + (16 * s + col) * T::RP + 32 * kk + 8 * g);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, oreg[kk], dp, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kj = k0 + 16 * s + 4 * g + i;
          const bool ok = FULL || (kj < N && query < N && (!CAUSAL || kj <= query));
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cl2e, -Lq));
          const float p = ok ? e : 0.0f;
          dS[s][i] = p * (dp[i] - Dq);
          smax = fmaxf(smax, fabsf(dS[s][i]));
        }
      }
      smax = xg_max(smax);
      const v4i aS = codes16(dS, smax > 0.0f ? div_rn(127.0f, smax) : 0.0f);
      const float sS = smax > 0.0f ? div_rn(smax, 127.0f) : 0.0f;
      float rS[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rS[i] = __shfl(sS, 4 * g + i);
#pragma unroll
      for (int n = 0; n < T::NN; ++n) {
        const v4i bk = *reinterpret_cast<const v4i*>(sK8 + (16 * n + col) * T::CP + 16 * g);
        const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(aS, bk, v4i{0, 0, 0, 0}, 0, 0, 0);
        const float ck = sKs[16 * n + col];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] = __builtin_fmaf((float)r[i], rS[i] * ck, acc[n][i]);
      }
    };
    if (full) tile(std::true_type{});
    else tile(std::false_type{});
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qr = qb * BB + wave * 16 + 4 * g + i;
    if (qr >= N) continue;
#pragma unroll
    for (int n = 0; n < T::NN; ++n) store_out<OUT_F32>(dq, (bh * N + qr) * D + 16 * n + col, c * acc[n][i]);
  }
}

// ---------------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------------
namespace {
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
}  // namespace

enum { BWD_PREP = 1, BWD_DKDV = 2, BWD_DQ = 4 };

// Workspace layout (offsets in bytes, each 256-aligned; Np = ceil(N/64)*64, nb = Np/64):
//   Q^ bf16 [BH,N,D] | K^ bf16 [BH,N,D] | Q8, K8, dO8 int8 [BH,D,Np] each |
//   Q8, K8, dO8 scales fp32 [BH,D,nb] each | D fp32 [BH,N]
struct BwdWs {
  int64_t qh, kh, q8, k8, do8, q8s, k8s, do8s, dl, total;
};

BwdWs bwd_ws_layout(int64_t BH, int N, int D) {
  const int64_t Np = ((int64_t)N + BB - 1) / BB * BB, nb = Np / BB;
  BwdWs w;
  int64_t off = 0;
  w.qh = off; off += align256(BH * N * D * 2);
  w.kh = off; off += align256(BH * N * D * 2);
  w.q8 = off; off += align256(BH * D * Np);
  w.k8 = off; off += align256(BH * D * Np);
  w.do8 = off; off += align256(BH * D * Np);
  w.q8s = off; off += align256(BH * D * nb * 4);
  w.k8s = off; off += align256(BH * D * nb * 4);
  w.do8s = off; off += align256(BH * D * nb * 4);
  w.dl = off; off += align256(BH * N * 4);
  w.total = off;
  return w;
}

size_t bwd_workspace_bytes(int64_t BH, int N, int D) { return (size_t)bwd_ws_layout(BH, N, D).total; }

template <int D>
static hipError_t launch_bwd_d(int stages, bool mx, const void* qc, const void* qs, const void* kc, const void* ks,
                               const void* v, const void* o, const void* dout, const float* lse, int BH, int N,
                               bool causal, float c, void* dq, void* dk, void* dv, bool out_f32, void* ws,
                               hipStream_t st) {
  const BwdWs L = bwd_ws_layout(BH, N, D);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  __bf16* qh = reinterpret_cast<__bf16*>(base + L.qh);
  __bf16* kh = reinterpret_cast<__bf16*>(base + L.kh);
  int8_t* q8 = reinterpret_cast<int8_t*>(base + L.q8);
  int8_t* k8 = reinterpret_cast<int8_t*>(base + L.k8);
  int8_t* do8 = reinterpret_cast<int8_t*>(base + L.do8);
  float* q8s = reinterpret_cast<float*>(base + L.q8s);
  float* k8s = reinterpret_cast<float*>(base + L.k8s);
  float* do8s = reinterpret_cast<float*>(base + L.do8s);
  float* dl = reinterpret_cast<float*>(base + L.dl);
  const int Np = (N + BB - 1) / BB * BB, nb = Np / BB;
  const dim3 pg(nb, BH);
  const uint8_t* qcb = reinterpret_cast<const uint8_t*>(qc);
  const uint8_t* qsb = reinterpret_cast<const uint8_t*>(qs);
  const uint8_t* kcb = reinterpret_cast<const uint8_t*>(kc);
  const uint8_t* ksb = reinterpret_cast<const uint8_t*>(ks);
  const f16* vh = reinterpret_cast<const f16*>(v);
  const f16* oh = reinterpret_cast<const f16*>(o);
  const f16* doh = reinterpret_cast<const f16*>(dout);
  if (stages & BWD_PREP) {
    if (mx) {
      bwd_prep_kernel<D, 1><<<pg, 256, 0, st>>>(qcb, qsb, nullptr, nullptr, N, Np, qh, q8, q8s, nullptr);
      bwd_prep_kernel<D, 1><<<pg, 256, 0, st>>>(kcb, ksb, nullptr, nullptr, N, Np, kh, k8, k8s, nullptr);
    } else {
      bwd_prep_kernel<D, 0><<<pg, 256, 0, st>>>(qcb, qsb, nullptr, nullptr, N, Np, qh, q8, q8s, nullptr);
      bwd_prep_kernel<D, 0><<<pg, 256, 0, st>>>(kcb, ksb, nullptr, nullptr, N, Np, kh, k8, k8s, nullptr);
    }
    bwd_prep_kernel<D, 2><<<pg, 256, 0, st>>>(nullptr, nullptr, doh, oh, N, Np, nullptr, do8, do8s, dl);
  }
  const int grid = BH * nb;
#define SAGE_BWD_LAUNCH(CZ, F32)                                                                          \
  do {                                                                                                    \
    if (stages & BWD_DKDV)                                                                                \
      bwd_dkdv_kernel<D, CZ, F32><<<grid, 256, 0, st>>>(qh, kh, vh, doh, q8, q8s, do8, do8s, lse, dl, N, Np, \
                                                        BH, c, dk, dv);                                   \
    if (stages & BWD_DQ)                                                                                  \
      bwd_dq_kernel<D, CZ, F32><<<grid, 256, 0, st>>>(qh, kh, vh, doh, k8, k8s, lse, dl, N, Np, BH, c, dq); \
  } while (0)
  if (causal) {
    if (out_f32) SAGE_BWD_LAUNCH(true, true);
    else SAGE_BWD_LAUNCH(true, false);
  } else {
    if (out_f32) SAGE_BWD_LAUNCH(false, true);
    else SAGE_BWD_LAUNCH(false, false);
  }
#undef SAGE_BWD_LAUNCH
  return hipGetLastError();
}

// stages: a mask of BWD_PREP (the three operand preparations), BWD_DKDV and BWD_DQ, launched in
// that order; the gradient stages read what the preparation left in the workspace.
hipError_t launch_attn_bwd(int stages, bool mx, const void* qc, const void* qs, const void* kc, const void* ks,
                           const void* v, const void* o, const void* dout, const float* lse, int BH, int N, int D,
                           bool causal, float c, void* dq, void* dk, void* dv, bool out_f32, void* ws,
                           hipStream_t st) {
  if (D == 64)
    return launch_bwd_d<64>(stages, mx, qc, qs, kc, ks, v, o, dout, lse, BH, N, causal, c, dq, dk, dv, out_f32, ws, st);
  return launch_bwd_d<128>(stages, mx, qc, qs, kc, ks, v, o, dout, lse, BH, N, causal, c, dq, dk, dv, out_f32, ws, st);
}

}  // namespace sage
