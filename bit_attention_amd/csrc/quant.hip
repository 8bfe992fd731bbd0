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

// V: one workgroup per (batch*head, run of `tpw` <= 4 consecutive 128-token tiles). Each tile, a
// contiguous D*256-byte run of fp16, is loaded into registers with 16-byte loads while the
// previous tile is encoded, then staged in LDS (row pitch D+8 halves keeps 16-byte alignment).
// Item (channel d, block) gathers its values in slot order from LDS; the blocks of a channel sit
// in consecutive lanes, so their code bytes form one contiguous run per channel. Four blocks'
// scale bytes are gathered into one dword per tile, and after the run the lane of block 0 stores
// the channel's scale bytes of all the run's tiles together. Token positions >= N are zero.
// FMT 0: NVFP4 (16-slot blocks, E4M3 scale of amax/6); 1: MXFP4 (32-slot blocks, E8M0 scale;
// codes are the E2M1 value nearest the exact quotient, ties to even); 2: MXFP8 (32-slot blocks;
// codes the E4M3 value nearest x / 2^X, ties to even, clamped to +-448; sign the input's).
template <int D, int FMT>
__global__ __launch_bounds__(256) void quant_v_tile_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales, int N, int64_t Np, int tpw) {
  constexpr bool F8 = FMT == 2;
  constexpr int PITCH = D + 8;  // halves
  constexpr int BLK = FMT == 0 ? 16 : 32, NB = KV_TILE / BLK;
  constexpr int CPB = F8 ? BLK : BLK / 2;  // code bytes per block
  constexpr int PPT = KV_TILE * D / 8 / 256;  // 16-byte pieces of a tile per thread
  __shared__ __attribute__((aligned(16))) __half tile[KV_TILE * PITCH];
  const int64_t bh = blockIdx.y;
  const int ntiles = (int)(Np / KV_TILE);
  const int kt0 = blockIdx.x * tpw, kt1 = min(ntiles, kt0 + tpw);
  uint4 pre[PPT];
  // scale dwords of this thread's items, one per tile of the run (tpw <= 4, see v_tiles_per_wg),
  // stored once at the end so that each channel's scale bytes of the run leave as one burst
  constexpr int ITEMS = D * NB / 256;
  unsigned sacc[ITEMS][4] = {};
  // the tile's fp16 pieces into registers (token positions >= N read as zero)
  auto load = [&](int kt) {
    const int tok0 = kt * KV_TILE, ntok = min(KV_TILE, N - tok0);
    const uint4* xs = reinterpret_cast<const uint4*>(x + (bh * N + tok0) * (int64_t)D);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int e = threadIdx.x + 256 * i, tok = e / (D / 8);
      pre[i] = tok < ntok ? xs[e] : make_uint4(0, 0, 0, 0);
    }
  };
  load(kt0);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int tix = kt - kt0;
    __syncthreads();  // the previous tile's LDS reads are complete
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int e = threadIdx.x + 256 * i, tok = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<uint4*>(&tile[tok * PITCH + 8 * c8]) = pre[i];
    }
    __syncthreads();
    if (kt + 1 < kt1) load(kt + 1);  // in flight while this tile is encoded and stored
    static_assert((D * NB) % 256 == 0, "every lane of a quad takes part in each pass");
#pragma unroll
    for (int ii = 0; ii < ITEMS; ++ii) {
      const int it = threadIdx.x + 256 * ii;
      const int d = it / NB, blk = it % NB;
      float v[BLK];
#pragma unroll
      for (int u = 0; u < BLK; ++u) v[u] = (float)tile[slot_token(blk * BLK + u) * PITCH + d];
      float amax = 0.0f;
#pragma unroll
      for (int u = 0; u < BLK; ++u) amax = fmaxf(amax, fabsf(v[u]));
      float s;
      const unsigned sb = FMT == 2 ? mx8_scale(amax, &s) : FMT == 1 ? mx_scale(amax, &s) : nv_scale(amax, &s);
      unsigned words[CPB / 4];
      if (F8) {
        const float r = s > 0.0f ? as_f((unsigned)(254 - (int)sb) << 23) : 0.0f;  // 1/s, exact
#pragma unroll
        for (int w = 0; w < CPB / 4; ++w) {
          float q[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_fmed3f(v[4 * w + k] * r, -448.0f, 448.0f);
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
          words[w] = (unsigned)word;
        }
      } else {
        encode_block<BLK>(v, s, FMT == 1, words);
      }
      uint4* crow = reinterpret_cast<uint4*>(codes + (bh * D + d) * (F8 ? Np : Np / 2) +
                                             (int64_t)kt * (F8 ? KV_TILE : KV_TILE / 2) + blk * CPB);
      if (CPB == 8) {
        *reinterpret_cast<uint2*>(crow) = make_uint2(words[0], words[CPB / 4 > 1 ? 1 : 0]);
      } else {
#pragma unroll
        for (int q = 0; q < CPB / 16; ++q)
          crow[q] = make_uint4(words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]);
      }
      // four consecutive blocks' scale bytes, gathered into the lane of the first
      const unsigned s1 = __shfl_down(sb, 1, 4), s2 = __shfl_down(sb, 2, 4), s3 = __shfl_down(sb, 3, 4);
      const unsigned wv = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u == tix) sacc[ii][u] = wv;
    }
  }
  // the run's scale bytes of each channel are contiguous: NB bytes per tile. NVFP4 (NB = 8):
  // the lane of blocks 0..3 takes the partner dword (blocks 4..7) from the lane 4 above it.
  const int nt = kt1 - kt0;
#pragma unroll
  for (int ii = 0; ii < ITEMS; ++ii) {
    const int it = threadIdx.x + 256 * ii;
    const int d = it / NB, blk = it % NB;
    unsigned w[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (NB == 8) {
        const unsigned hi = __shfl_down(sacc[ii][u], 4, 8);
        w[2 * u] = sacc[ii][u]; w[2 * u + 1] = hi;
      } else {
        w[u] = sacc[ii][u];
      }
    }
    if (blk == 0) {
      uint8_t* dst = scales + (bh * D + d) * (Np / BLK) + (int64_t)kt0 * NB;
      const int nw = nt * NB / 4;  // dwords to store
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < nw) reinterpret_cast<unsigned*>(dst)[q] = w[q];
    }
  }
}

// tiles per workgroup of the V quantiser: up to 4, keeping at least 2048 workgroups
inline int v_tiles_per_wg(int64_t ntiles, int BH) {
  int tpw = 4;
  while (tpw > 1 && ((ntiles + tpw - 1) / tpw) * BH < 2048) tpw /= 2;
  return tpw;
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
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE, nt = Np / KV_TILE;
  const int tpw = v_tiles_per_wg(nt, BH);
  const dim3 grid((unsigned)((nt + tpw - 1) / tpw), (unsigned)BH), block(256);
  if (D == 64) quant_v_tile_kernel<64, 2><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, N, Np, tpw);
  else quant_v_tile_kernel<128, 2><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, N, Np, tpw);
  return hipGetLastError();
}

hipError_t launch_quant_v(bool mx, const void* x, int BH, int N, int D, void* codes, void* scales, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const __half* xp = (const __half*)x;
  uint8_t *c = (uint8_t*)codes, *s = (uint8_t*)scales;
  const int64_t nt = Np / KV_TILE;
  const int tpw = v_tiles_per_wg(nt, BH);
  const dim3 grid((unsigned)((nt + tpw - 1) / tpw), (unsigned)BH), block(256);
  if (mx) {
    if (D == 64) quant_v_tile_kernel<64, 1><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw);
    else quant_v_tile_kernel<128, 1><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw);
  } else {
    if (D == 64) quant_v_tile_kernel<64, 0><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw);
    else quant_v_tile_kernel<128, 0><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw);
  }
  return hipGetLastError();
}

}  // namespace sage
