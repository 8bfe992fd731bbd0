// quant.hip — FP4 microscaling quantisation kernels (Q, K along D; V along tokens in slot
// order), NVFP4 (1x16, E4M3 scale) and MXFP4 (1x32, E8M0 scale); and MXFP8 V (E4M3 elements,
// 1x32, E8M0 scale) for the variant with FP8 P and V.
//
// SageAttention3 (arXiv 2505.11594), DeepTech article: both matmuls of attention take FP4
// operands quantised in 1x16 groups (section on the two FP4 obstacles); NVFP4 is E2M1 with an
// E4M3 scale per 16 values, MXFP4 E2M1 with an E8M0 scale per 32 (section on FP4 data types);
// the quantisation kernel also produces the permuted key order the attention kernel's register
// layout needs (section on the hardware implementation).
//
// Bound: HBM. One pass: 2 B/element read, 0.5 B codes + 1/16 (1/32) B scales written.
#include "device.h"

namespace sage {

// Codes of n values with block scale s (E4M3 value or power of two): the E2M1 value nearest the
// exact quotient x/s, ties to even. q = x*r (r = 1/s rounded) is refined by one Newton step on
// the exact remainder; the refined q equals x/s exactly whenever x/s is a tie point, and is
// within 2^-45 relative otherwise, while a non-tie fp16 x is at least 2^-12 relative away from
// any tie, so the hardware's round-to-nearest-even conversion then decides correctly.
// The sum in the last step turns a -0 quotient into +0, so the input's sign is put back (the
// code's sign bit is the input's, -0 included).
__device__ __forceinline__ float refine_quot(float x, float s, float r) {
  float q = x * r;
  float rem = __builtin_fmaf(-s, q, x);
  return __builtin_copysignf(__builtin_fmaf(rem, r, q), x);
}

template <int BLK>
__device__ __forceinline__ void encode_block(const float* v, float s, bool pow2_scale, unsigned* out_words) {
  const float r = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
#pragma unroll
  for (int w = 0; w < BLK / 8; ++w) {
    unsigned word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float x0 = v[8 * w + 2 * b], x1 = v[8 * w + 2 * b + 1];
      float q0, q1;
      if (pow2_scale) { q0 = x0 * r; q1 = x1 * r; }  // exact
      else { q0 = refine_quot(x0, s, r); q1 = refine_quot(x1, s, r); }
      switch (b) {
        case 0: word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, 0); break;
        case 1: word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, 1); break;
        case 2: word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, 2); break;
        default: word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, 3); break;
      }
    }
    out_words[w] = word;
  }
}

// NVFP4 scale byte and value of a block with absolute maximum amax (exact FP32).
__device__ __forceinline__ unsigned nv_scale(float amax, float* s) {
  const unsigned b = e4m3_encode(__fdiv_rn(amax, 6.0f));
  *s = e4m3_decode(b);
  return b;
}

// MXFP4 scale byte of a block with absolute maximum amax (finite, amax < 2^127): the OCP rule
// 2^(floor(log2 amax) - 2); byte 0 for amax == 0.
__device__ __forceinline__ unsigned mx_scale(float amax, float* s) {
  if (!(amax > 0.0f)) { *s = 0.0f; return 0u; }
  int e = (int)((as_u(amax) >> 23) & 0xFF);            // biased exponent (0: subnormal)
  int fl = e ? e - 127 : (-127 - __builtin_clz(as_u(amax) & 0x7FFFFFu) + 9);  // floor(log2)
  int X = fl - 2;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  *s = X >= -126 ? as_f((unsigned)(X + 127) << 23) : as_f(1u << (X + 149));  // 2^X, exact
  return (unsigned)(X + 127);
}

// MXFP8 scale byte: the OCP rule 2^(floor(log2 amax) - 8) (8 = the largest E4M3 exponent);
// byte 0 and s = 0 for amax == 0. amax is an fp16 magnitude here, so 2^X is a normal float.
__device__ __forceinline__ unsigned mx8_scale(float amax, float* s) {
  if (!(amax > 0.0f)) { *s = 0.0f; return 0u; }
  const int X = (int)((as_u(amax) >> 23) & 0xFF) - 127 - 8;
  *s = as_f((unsigned)(X + 127) << 23);
  return (unsigned)(X + 127);
}

template <int BLK>
__device__ __forceinline__ void load_f16(const __half* p, float* v) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int w = 0; w < BLK / 8; ++w) {
    uint4 u = q[w];
    const unsigned ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * w + 2 * k] = (float)__ushort_as_half((unsigned short)(ww[k] & 0xFFFF));
      v[8 * w + 2 * k + 1] = (float)__ushort_as_half((unsigned short)(ww[k] >> 16));
    }
  }
}

// Q and K: one thread per block of BLK consecutive channels. Blocks of consecutive threads are
// contiguous in memory, so loads and stores coalesce.
template <int BLK, bool MX>
__global__ __launch_bounds__(256) void quant_rows_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[BLK];
  load_f16<BLK>(x + b * BLK, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < BLK; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float s;
  const unsigned sb = MX ? mx_scale(amax, &s) : nv_scale(amax, &s);
  unsigned words[BLK / 8];
  encode_block<BLK>(v, s, MX, words);
  if (BLK == 16) {
    reinterpret_cast<uint2*>(codes)[b] = make_uint2(words[0], words[1]);
  } else {
    reinterpret_cast<uint4*>(codes)[b] = make_uint4(words[0], words[1], words[BLK / 8 > 2 ? 2 : 0], words[BLK / 8 > 3 ? 3 : 0]);
  }
  scales[b] = (uint8_t)sb;
}

// V, MXFP4: one workgroup per (batch*head, 128-token tile). The tile is staged in LDS (row pitch
// D+2 halves to spread banks), then each thread quantises (channel, block) items whose 32 values
// are gathered in slot order; with 32-value blocks this beats the register gather below, whose
// blocks would need more registers than four waves per SIMD allow. Token positions >= N are zero.
template <int D, int BLK, bool MX>
__global__ __launch_bounds__(256) void quant_v_lds_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, int N, int64_t Np) {
  constexpr int PITCH = D + 2;
  __shared__ __attribute__((aligned(16))) __half tile[KV_TILE * PITCH];
  const int kt = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tok0 = kt * KV_TILE;
  const __half* xs = x + (bh * N + tok0) * (int64_t)D;
  const int ntok = min(KV_TILE, N - tok0);
  // stage: 4-byte granules (pairs of halves), coalesced over the contiguous tile
  for (int e = threadIdx.x; e < KV_TILE * D / 2; e += blockDim.x) {
    const int tok = e / (D / 2), c2 = e % (D / 2);
    unsigned u = 0;
    if (tok < ntok) u = reinterpret_cast<const unsigned*>(xs)[(int64_t)tok * (D / 2) + c2];
    *reinterpret_cast<unsigned*>(&tile[tok * PITCH + 2 * c2]) = u;
  }
  __syncthreads();
  constexpr int NB = KV_TILE / BLK;  // blocks per channel per tile
  for (int it = threadIdx.x; it < D * NB; it += blockDim.x) {
    const int d = it / NB, blk = it % NB;
    float v[BLK];
#pragma unroll
    for (int u = 0; u < BLK; ++u) v[u] = (float)tile[slot_token(blk * BLK + u) * PITCH + d];
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < BLK; ++u) amax = fmaxf(amax, fabsf(v[u]));
    float s;
    const unsigned sb = MX ? mx_scale(amax, &s) : nv_scale(amax, &s);
    unsigned words[BLK / 8];
    encode_block<BLK>(v, s, MX, words);
    uint8_t* crow = codes + (bh * D + d) * (Np / 2) + (int64_t)kt * (KV_TILE / 2) + blk * (BLK / 2);
    if (BLK == 16) *reinterpret_cast<uint2*>(crow) = make_uint2(words[0], words[1]);
    else *reinterpret_cast<uint4*>(crow) = make_uint4(words[0], words[1], words[BLK / 8 > 2 ? 2 : 0], words[BLK / 8 > 3 ? 3 : 0]);
    scales[(bh * D + d) * (Np / BLK) + (int64_t)kt * NB + blk] = (uint8_t)sb;
  }
}

// V, MXFP8: the workgroup layout of quant_v_lds_kernel; each (channel, block) item writes its 32
// E4M3 bytes. The quotient x / 2^X is exact (a power-of-two scale); quotients beyond +-448 clamp
// to +-448 before the hardware's round-to-nearest-even conversion; the sign is the input's.
template <int D>
__global__ __launch_bounds__(256) void quant_v8_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int N, int64_t Np) {
  constexpr int PITCH = D + 2;
  constexpr int BLK = 32, NB = KV_TILE / BLK;
  __shared__ __attribute__((aligned(16))) __half tile[KV_TILE * PITCH];
  const int kt = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tok0 = kt * KV_TILE;
  const __half* xs = x + (bh * N + tok0) * (int64_t)D;
  const int ntok = min(KV_TILE, N - tok0);
  for (int e = threadIdx.x; e < KV_TILE * D / 2; e += blockDim.x) {
    const int tok = e / (D / 2), c2 = e % (D / 2);
    unsigned u = 0;
    if (tok < ntok) u = reinterpret_cast<const unsigned*>(xs)[(int64_t)tok * (D / 2) + c2];
    *reinterpret_cast<unsigned*>(&tile[tok * PITCH + 2 * c2]) = u;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < D * NB; it += blockDim.x) {
    const int d = it / NB, blk = it % NB;
    float v[BLK];
#pragma unroll
    for (int u = 0; u < BLK; ++u) v[u] = (float)tile[slot_token(blk * BLK + u) * PITCH + d];
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < BLK; ++u) amax = fmaxf(amax, fabsf(v[u]));
    float s;
    const unsigned sb = mx8_scale(amax, &s);
    const float r = s > 0.0f ? as_f((unsigned)(254 - (int)sb) << 23) : 0.0f;  // 1/s, exact
    unsigned words[BLK / 4];
#pragma unroll
    for (int w = 0; w < BLK / 4; ++w) {
      float q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_fmed3f(v[4 * w + k] * r, -448.0f, 448.0f);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
      words[w] = (unsigned)word;
    }
    uint4* crow = reinterpret_cast<uint4*>(codes + (bh * D + d) * Np + (int64_t)kt * KV_TILE + blk * BLK);
    crow[0] = make_uint4(words[0], words[1], words[2], words[3]);
    crow[1] = make_uint4(words[4], words[5], words[6], words[7]);
    scales[(bh * D + d) * (Np / BLK) + (int64_t)kt * NB + blk] = (uint8_t)sb;
  }
}

// V, NVFP4: one wave per (batch*head, pair of 128-token tiles). Each lane owns a channel pair; with
// D = 128 the 64 lanes cover all channels and walk the two tiles in turn, with D = 64 each half
// of the wave takes one tile. A token's channels are read by the lanes of that tile together
// (one contiguous row per load), so the gather into slot order needs no LDS: a lane reads its
// two channels token by token in the order the blocks take them. Each lane then writes its
// channels' 64 code bytes per tile (a tile pair's 128 bytes come from one wave) and their scale
// bytes. Token positions >= N are zero.
template <int D, int BLK, bool MX>
__global__ __launch_bounds__(256) void quant_v_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, int N, int64_t Np,
                                                      int npairs, int nwaves) {
  constexpr int LPT = D / 2;            // lanes per tile (one channel pair each)
  constexpr int PASSES = LPT / 32;      // tiles of the pair walked in turn: 2 (D = 128) or 1
  constexpr int NB = KV_TILE / BLK;     // blocks per channel per tile
  constexpr int WPB = BLK / 8;          // code dwords per block
  const int lane = threadIdx.x & 63;
  const int wv = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (wv >= nwaves) return;  // whole waves only; the kernel has no barrier
  const int64_t bh = wv / npairs;
  const int pr = wv % npairs;
  const int ntiles = (int)(Np / KV_TILE);
  const int d0 = 2 * (lane % LPT);
  const __half* xs = x + bh * N * (int64_t)D + d0;
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    const int kt = 2 * pr + (PASSES == 2 ? pass : lane / LPT);
    if (kt >= ntiles) break;
    const int tok0 = kt * KV_TILE;
    unsigned cw[2][NB * WPB];
    unsigned sbytes[2][NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      float v[2][BLK];
#pragma unroll
      for (int u = 0; u < BLK; ++u) {
        const int tok = tok0 + slot_token(blk * BLK + u);
        unsigned bits = 0;
        if (tok < N) bits = *reinterpret_cast<const unsigned*>(xs + (int64_t)tok * D);
        v[0][u] = (float)__ushort_as_half((unsigned short)(bits & 0xFFFF));
        v[1][u] = (float)__ushort_as_half((unsigned short)(bits >> 16));
      }
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < BLK; ++u) amax = fmaxf(amax, fabsf(v[ch][u]));
        float sc;
        sbytes[ch][blk] = MX ? mx_scale(amax, &sc) : nv_scale(amax, &sc);
        encode_block<BLK>(v[ch], sc, MX, &cw[ch][blk * WPB]);
      }
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int64_t row = bh * D + d0 + ch;
      uint4* crow = reinterpret_cast<uint4*>(codes + row * (Np / 2) + (int64_t)kt * (KV_TILE / 2));
#pragma unroll
      for (int q = 0; q < 4; ++q) crow[q] = make_uint4(cw[ch][4 * q], cw[ch][4 * q + 1], cw[ch][4 * q + 2], cw[ch][4 * q + 3]);
      uint8_t* srow = scales + row * (Np / BLK) + (int64_t)kt * NB;
      if (NB == 8) {
        *reinterpret_cast<uint2*>(srow) =
            make_uint2(sbytes[ch][0] | sbytes[ch][1] << 8 | sbytes[ch][2] << 16 | sbytes[ch][3] << 24,
                       sbytes[ch][NB > 4 ? 4 : 0] | sbytes[ch][NB > 5 ? 5 : 0] << 8 |
                           sbytes[ch][NB > 6 ? 6 : 0] << 16 | sbytes[ch][NB > 7 ? 7 : 0] << 24);
      } else {
        *reinterpret_cast<unsigned*>(srow) = sbytes[ch][0] | sbytes[ch][1] << 8 | sbytes[ch][2] << 16 | sbytes[ch][3] << 24;
      }
    }
  }
}

// ---- launchers (arguments already validated by the C ABI layer) ----
hipError_t launch_quant_rows(bool mx, const void* x, int64_t rows, int D, void* codes, void* scales, hipStream_t st) {
  const int blk = mx ? 32 : 16;
  const int64_t nblocks = rows * (D / blk);
  const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
  if (mx) quant_rows_kernel<32, true><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, nblocks);
  else quant_rows_kernel<16, false><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_quant_v8(const void* x, int BH, int N, int D, void* codes, void* scales, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const dim3 grid((unsigned)(Np / KV_TILE), (unsigned)BH), block(256);
  if (D == 64) quant_v8_kernel<64><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, N, Np);
  else quant_v8_kernel<128><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, N, Np);
  return hipGetLastError();
}

hipError_t launch_quant_v(bool mx, const void* x, int BH, int N, int D, void* codes, void* scales, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const __half* xp = (const __half*)x;
  uint8_t *c = (uint8_t*)codes, *s = (uint8_t*)scales;
  if (mx) {
    const dim3 grid((unsigned)(Np / KV_TILE), (unsigned)BH), block(256);
    if (D == 64) quant_v_lds_kernel<64, 32, true><<<grid, block, 0, st>>>(xp, c, s, N, Np);
    else quant_v_lds_kernel<128, 32, true><<<grid, block, 0, st>>>(xp, c, s, N, Np);
  } else {
    const int npairs = (int)((Np / KV_TILE + 1) / 2);
    const int nwaves = BH * npairs;
    const dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
    if (D == 64) quant_v_kernel<64, 16, false><<<grid, block, 0, st>>>(xp, c, s, N, Np, npairs, nwaves);
    else quant_v_kernel<128, 16, false><<<grid, block, 0, st>>>(xp, c, s, N, Np, npairs, nwaves);
  }
  return hipGetLastError();
}

}  // namespace sage
