// device.h — gfx950 device helpers for the FP4 attention kernels (GPU side only).
//
// Instruction semantics relied on (each checked on gfx950 against exhaustive or tie-point
// tables before use):
//   v_cvt_pk_fp8_f32          FP32 -> OCP E4M3, round to nearest even (overflow gives NaN, so
//                             callers clamp to 448 first)
//   v_cvt_f32_fp8             E4M3 -> FP32, exact
//   v_cvt_scalef32_pk_fp4_f32 two FP32 -> two E2M1 codes of x / 2^floor(log2 scale), round to
//                             nearest even, saturating at 6, sign kept (including -0)
//   v_cvt_scalef32_pk_f16_fp4 two E2M1 codes -> two fp16 values code * 2^floor(log2 scale)
//   v_exp_f32                 2^x within 1 ulp
//   MFMA layouts: 16x16xK: A/B lane l holds row/column l%16, K-chunk l/16 (8 halves for f16,
//   32 FP4 codes for the scaled FP4 form); C lane l holds rows 4(l/16)+i of column l%16.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int KV_TILE = 128;

// Token held by slot s of a 128-token tile: slot 32g + 4t + i holds token 16t + 4g + i. This is
// the key order in which a wave holds S^T after eight 16x16 MFMA subtiles (lane group g, subtile
// t, accumulator element i), so a lane's P values form whole blocks.
__host__ __device__ inline int slot_token(int s) { return 16 * ((s & 31) >> 2) + 4 * (s >> 5) + (s & 3); }

// Work item of workgroup L out of T. Workgroups are dispatched round-robin over the 8 XCDs
// (XCD x receives L = x, x + 8, ...); each XCD is given one contiguous range of work items, so
// the workgroups one XCD runs side by side share (batch, head), and with it K and V in that
// XCD's L2. A bijection of [0, T) for any T.
__device__ __forceinline__ int xcd_work(int L, int T) {
  const int x = L & 7, k = L >> 3, q = T >> 3, r = T & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

// Work item w of a causal launch -> (batch*head bh, query tile qt). Heads are taken in groups of
// G (the last group may be smaller); inside a group the heaviest query tiles (those with the most
// key tiles under the causal mask) of all its heads come first. Heavy and light items then mix
// along the grid, while one group's K and V stay small enough to share an XCD's L2 (the host
// picks G from the K/V bytes per head). G = 1 is head-major, heaviest tile first.
__device__ __forceinline__ void causal_work(int w, int nqt, int BH, int G, int64_t& bh, int& qt) {
  const int gsize = G * nqt, grp = w / gsize, base = grp * G;
  const int Gg = min(G, BH - base), r = w - grp * gsize;
  bh = base + r % Gg;
  qt = nqt - 1 - r / Gg;
}

// Heads per causal group (measured on B4 H32 N4096 and B1 H32 N32768): groups must not straddle
// the contiguous range of heads each XCD receives, so G is a power of two dividing the heads per
// XCD (BH / 8; 1 when BH is not a multiple of 8), at most 8, and small enough that the group's K
// and V (kv_bytes_per_head each) stay within 24 MiB.
inline int causal_group(int BH, int64_t kv_bytes_per_head) {
  if (BH % 8 != 0) return 1;
  const int hx = BH / 8;
  int64_t cap = (int64_t(24) << 20) / (kv_bytes_per_head > 0 ? kv_bytes_per_head : 1);
  if (cap > 8) cap = 8;
  int g = 1;
  while (2 * g <= hx && 2 * g <= cap && hx % (2 * g) == 0) g *= 2;
  return g;
}

__device__ __forceinline__ float as_f(unsigned u) { return __uint_as_float(u); }
__device__ __forceinline__ unsigned as_u(float f) { return __float_as_uint(f); }

// E4M3 byte of y (0 <= y, finite), round to nearest even, clamped to 448.
__device__ __forceinline__ unsigned e4m3_encode(float y) {
  y = fminf(y, 448.0f);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_decode(unsigned b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// 2^floor(log2 s) for s > 0 (s normal FP32), 1 for s == 0.
__device__ __forceinline__ float pow2_floor(float s) { return s > 0.0f ? as_f(as_u(s) & 0xFF800000u) : 1.0f; }

// max(a, b, c) in one v_max3_f32 (the compiler re-balances fmaxf trees into pairs otherwise).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max(a, b) in one v_max_f32. Without -fno-honor-nans the compiler quiets each operand that
// arrives as a bit pattern (a lane swap) first (v_max x, x, x), in case it is a signalling NaN;
// this form does not depend on that flag. Scores and their maxima never are NaN, so the plain
// instruction gives the same value.
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max over the lane pair {l, l^16}, over {l, l^32}, and over the four lanes {l, l^16, l^32,
// l^48} that share a column of a 16x16 MFMA tile (operands never NaN).
__device__ __forceinline__ float pair16_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u(v), as_u(v), false, false);
  return max2f(as_f(p[0]), as_f(p[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u(v), as_u(v), false, false);
  return max2f(as_f(r[0]), as_f(r[1]));
}
__device__ __forceinline__ float xg_max(float v) { return pair32_max(pair16_max(v)); }
__device__ __forceinline__ float xg_sum(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u(v), as_u(v), false, false);
  v = as_f(p[0]) + as_f(p[1]);
  auto r = __builtin_amdgcn_permlane32_swap(as_u(v), as_u(v), false, false);
  return as_f(r[0]) + as_f(r[1]);
}

// Two E2M1 codes (low byte of `byte2`) -> fp16 pair code * s, exact for E4M3 s: the hardware
// applies the power of two, the 1+m/8 mantissa is one exact fp16 multiply.
__device__ __forceinline__ v2h dequant2(unsigned byte2, float p2, v2h mu) {
  v2h h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(byte2, p2, 0);
  return h * mu;
}

// Eight E2M1 codes (one dword) times an fp16 scale pair, exact (an E4M3 scale times a code has at
// most 6 significant bits and lies in the normal fp16 range or is zero).
__device__ __forceinline__ v8h dequant8(unsigned w, v2h s) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E4M3 scale byte -> its value in fp16, exact (every E4M3 value is an fp16 value).
__device__ __forceinline__ _Float16 e4m3_to_f16(unsigned b) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false)[0];
}

}  // namespace sage
