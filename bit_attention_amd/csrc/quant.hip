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
// Bound: HBM. One pass: 2 B/element read, 0.5 B codes + 1/16 (1/32) B scales written; the NVFP4
// K and V kernels that also write K-hat / V-hat (exact fp16 dequantisation) add 2 B/element.
#include "device.h"

namespace sage {

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Codes of a block of values with scale s (E4M3 value or power of two): the E2M1 value nearest
// the exact quotient x/s, ties to even, the code's sign the input's (-0 included).
// Power of two: x * (1/s) is exact. E4M3 s: 1/s is split as r_hi + r_lo, r_hi the hardware
// reciprocal (within 1 ulp) scaled down by 2^-21, so that the residual e = 1 - s*r_hi is
// positive and exact in one fma (s has at most 4 significant bits), and r_lo = e*r_hi >= 0;
// r_hi + r_lo is 1/s within 2^-40 relative. q = fma(x, r_hi, x*r_lo) is then x/s within 2^-40
// before its one rounding: q equals x/s exactly when x/s is one of the tie points (0.25, 0.75,
// ..., 5), and otherwise x/s, with x fp16, is at least 2^-12 relative from every tie, so the
// hardware's round-to-nearest-even conversion of q decides as it would on x/s. For x = -0 both
// terms are -0 (r_hi, r_lo >= 0) and so is their sum. (An exhaustive check over every finite
// fp16 x and every positive E4M3 s, with the reciprocal off by one ulp either way, agrees.)
template <int BLK, typename Get>
__device__ __forceinline__ void encode_block(Get v, float s, bool pow2_scale, unsigned* out_words) {
  float rh, rl = 0.0f;
  if (pow2_scale) {
    // 1/s by exponent arithmetic: s = 2^X with X >= -26 for fp16 inputs (a normal float)
    rh = s > 0.0f ? as_f((254u << 23) - as_u(s)) : 0.0f;
  } else {
    rh = s > 0.0f ? __builtin_amdgcn_rcpf(s) * (1.0f - 0x1p-21f) : 0.0f;
    const float e = __builtin_fmaf(-s, rh, 1.0f);
    rl = s > 0.0f ? e * rh : 0.0f;
  }
#pragma unroll
  for (int w = 0; w < BLK / 8; ++w) {
    unsigned word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float x0 = v(8 * w + 2 * b), x1 = v(8 * w + 2 * b + 1);
      float q0, q1;
      if (pow2_scale) { q0 = x0 * rh; q1 = x1 * rh; }  // exact
      else { q0 = __builtin_fmaf(x0, rh, x0 * rl); q1 = __builtin_fmaf(x1, rh, x1 * rl); }
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

// NVFP4 scale byte and value of a block with absolute maximum amax (an fp16 magnitude): the
// E4M3 encoding of fl32(amax/6). The quotient is rounded correctly with one refinement step
// (Markstein): q0 = amax * fl32(1/6), the remainder amax - 6*q0 is exact in one fma, and
// q0 + remainder * fl32(1/6) rounds to fl32(amax/6) (checked exhaustively over fp16 amax).
__device__ __forceinline__ unsigned nv_scale(float amax, float* s) {
  constexpr float R6 = 1.0f / 6.0f;
  const float q0 = amax * R6;
  const float q = __builtin_fmaf(__builtin_fmaf(-6.0f, q0, amax), R6, q0);
  const unsigned b = e4m3_encode(q);
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

// One block of BLK consecutive channels at x: its codes and scale byte are stored at block index
// b; the code words are also returned (for a caller that dequantises them) with the scale byte.
template <int BLK, bool MX>
__device__ __forceinline__ unsigned quant_block(const __half* x, uint8_t* codes, uint8_t* scales, int64_t b,
                                                unsigned (&words)[BLK / 8]) {
  float v[BLK];
  load_f16<BLK>(x, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < BLK; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float s;
  const unsigned sb = MX ? mx_scale(amax, &s) : nv_scale(amax, &s);
  encode_block<BLK>([&](int u) { return v[u]; }, s, MX, words);
  if (BLK == 16) {
    reinterpret_cast<uint2*>(codes)[b] = make_uint2(words[0], words[1]);
  } else {
    reinterpret_cast<uint4*>(codes)[b] = make_uint4(words[0], words[1], words[BLK / 8 > 2 ? 2 : 0], words[BLK / 8 > 3 ? 3 : 0]);
  }
  scales[b] = (uint8_t)sb;
  return sb;
}

// Q and K: one thread per block of BLK consecutive channels. Blocks of consecutive threads are
// contiguous in memory, so loads and stores coalesce.
template <int BLK, bool MX>
__global__ __launch_bounds__(256) void quant_rows_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  unsigned words[BLK / 8];
  quant_block<BLK, MX>(x + b * BLK, codes, scales, b, words);
}

// NVFP4 K together with K-hat, its exact fp16 dequantisation ([BH][Np][D], rows >= N zero), the
// layout the attention copies K tiles from. Grid (ceil(Np*D/16 / 256), BH): one thread per
// 16-channel block of a head's padded rows. Codes and scales are those of quant_rows_kernel;
// each K-hat value is its code times the block's E4M3 scale.
template <int D>
__global__ __launch_bounds__(256) void quant_k_hat_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int N, int64_t Np,
                                                          _Float16* __restrict__ kh) {
  constexpr int BPR = D / 16;  // blocks per row
  const int64_t bh = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // block within the head's padded rows
  if (i >= Np * BPR) return;
  const int64_t j = i / BPR;
  v8h lo = v8h{0, 0, 0, 0, 0, 0, 0, 0}, hi = lo;
  if (j < N) {
    const int64_t b = (bh * N + j) * BPR + i % BPR;
    unsigned words[2];
    const unsigned sb = quant_block<16, false>(x + b * 16, codes, scales, b, words);
    const _Float16 sh = e4m3_to_f16(sb);
    lo = dequant8(words[0], v2h{sh, sh});
    hi = dequant8(words[1], v2h{sh, sh});
  }
  v8h* dst = reinterpret_cast<v8h*>(kh + bh * Np * D + i * 16);
  dst[0] = lo;
  dst[1] = hi;
}

// V: one workgroup of 2*D threads per (batch*head, run of `tpw` consecutive 128-token tiles).
// Each tile, a contiguous D*256-byte run of fp16, is loaded into registers with 16-byte loads,
// two tiles ahead (two register buffers, each refilled as soon as it is staged), then staged in
// LDS (row pitch D+8 halves keeps 16-byte alignment). An item is (channel pair dp, block): it
// reads its block's slots as 32-bit words (channels 2dp and 2dp+1 of one token) and encodes the
// two channels' blocks. Lane l of wave w takes channel pair 16w + l%16 and block l/16 (NVFP4:
// blocks 2(l/16) and 2(l/16)+1 in two passes), so the 64 lanes of one LDS read touch 16
// consecutive words in each of 4 token rows whose word offsets differ by multiples of 16
// modulo 64: no bank conflicts. Codes and scales are stored tile by tile ([B,H,Np/128,D,64]
// and [B,H,Np/128,D,128/blk]; MXFP8 codes [B,H,Np/128,D,128]): a lane stores 16 (MXFP8: 32)
// contiguous code bytes of each of its two channels, which complete whole 128-byte lines
// within one tile, and lanes gather a channel's scale bytes with shuffles so that each wave
// stores one contiguous run of them. Token positions >= N are zero.
// FMT 0: NVFP4 (16-slot blocks, E4M3 scale of amax/6); 1: MXFP4 (32-slot blocks, E8M0 scale;
// codes are the E2M1 value nearest the exact quotient, ties to even); 2: MXFP8 (32-slot blocks;
// codes the E4M3 value nearest x / 2^X, ties to even, clamped to +-448; sign the input's).
// HAT (NVFP4 only): V-hat, each code times its block's E4M3 scale in fp16, is also stored in the
// codes' layout ([B,H,Np/128,D,128] halves), from the code words and scale bytes just made.
template <int D, int FMT, bool HAT = false>
__global__ __launch_bounds__(2 * D, FMT == 2 ? 2 : 3) void quant_v_tile_kernel(const __half* __restrict__ x, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, int N, int64_t Np, int tpw,
                                                             _Float16* __restrict__ vh) {
  constexpr bool F8 = FMT == 2, NV = FMT == 0;
  static_assert(!HAT || NV, "V-hat is written for NVFP4 only");
  constexpr int NT = 2 * D;     // threads: one channel pair x one block (pair) each
  constexpr int PITCH = D + 8;  // halves
  constexpr int BLK = NV ? 16 : 32, NB = KV_TILE / BLK;
  constexpr int PASSES = NV ? 2 : 1;
  constexpr int LW = F8 ? 8 : 4;             // code dwords per lane, channel and tile (16 or 32 bytes)
  constexpr int PPT = KV_TILE * D / 8 / NT;  // 16-byte pieces of a tile per thread
  constexpr int64_t TB = F8 ? KV_TILE : KV_TILE / 2;  // code bytes per channel and tile
  static_assert(NT % 64 == 0 && D / 32 == NT / 64, "one wave per group of 16 channel pairs");
  __shared__ __attribute__((aligned(16))) __half tile[KV_TILE * PITCH];
  const int64_t bh = blockIdx.y;
  const int ntiles = (int)(Np / KV_TILE);
  const int kt0 = blockIdx.x * tpw, kt1 = min(ntiles, kt0 + tpw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int dp = 16 * (tid >> 6) + (lane & 15), j = lane >> 4;
  // codes are stored tile by tile ([Np/128][D][TB]): this lane's 16 (MXFP8: 32) bytes of
  // channel 2dp of tile kt sit at ((bh*ntiles + kt)*D + 2dp)*TB + that width times j
  uint8_t* cbase = codes + (bh * ntiles * D + 2 * dp) * TB + (F8 ? 32 : 16) * j;
  auto load = [&](int kt, uint4 (&buf)[PPT]) {
    const int tok0 = kt * KV_TILE, ntok = min(KV_TILE, N - tok0);
    const uint4* xs = reinterpret_cast<const uint4*>(x + (bh * N + tok0) * (int64_t)D);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int e = tid + NT * i, tok = e / (D / 8);
      buf[i] = tok < ntok ? xs[e] : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_codes = [&](int kt, const unsigned (&wd)[2][LW]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint4* dst = reinterpret_cast<uint4*>(cbase + ((int64_t)kt * D + c) * TB);
#pragma unroll
      for (int q = 0; q < LW / 4; ++q) dst[q] = make_uint4(wd[c][4 * q], wd[c][4 * q + 1], wd[c][4 * q + 2], wd[c][4 * q + 3]);
    }
  };
  // One tile: stage `buf` in LDS, refill `buf` with tile ktn (if it is in the run) while this
  // tile is encoded, encode into wd and store the tile's scales.
  auto step = [&](int kt, uint4 (&buf)[PPT], int ktn, unsigned (&wd)[2][LW]) {
    __syncthreads();  // the previous tile's LDS reads are complete
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int e = tid + NT * i, tok = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<uint4*>(&tile[tok * PITCH + 8 * c8]) = buf[i];
    }
    if (ktn < kt1) load(ktn, buf);
    __syncthreads();
    unsigned sbp[PASSES];  // scale bytes per pass: channel 2dp in byte 0, 2dp+1 in byte 1
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int blk = NV ? 2 * j + ps : j;
      unsigned raw[BLK];
#pragma unroll
      for (int u = 0; u < BLK; ++u)
        raw[u] = *reinterpret_cast<const unsigned*>(&tile[slot_token(blk * BLK + u) * PITCH + 2 * dp]);
      // block maxima of both channels at once: fp16 magnitudes order as their 15-bit patterns
      v2u16 m2 = {0, 0};
#pragma unroll
      for (int u = 0; u < BLK; ++u) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(v2u16, raw[u] & 0x7FFF7FFFu));
      unsigned sbc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // element u of channel c, converted where it is used (halves are taken by shifts: a
        // bit cast of an element of a vector value reads element 0 with this compiler)
        auto v = [&](int u) { return (float)__ushort_as_half((unsigned short)(c ? raw[u] >> 16 : raw[u] & 0xFFFFu)); };
        const unsigned mm = __builtin_bit_cast(unsigned, m2);
        const float amax = (float)__ushort_as_half((unsigned short)(c ? mm >> 16 : mm & 0xFFFFu));
        float s;
        sbc[c] = FMT == 2 ? mx8_scale(amax, &s) : FMT == 1 ? mx_scale(amax, &s) : nv_scale(amax, &s);
        unsigned* out = &wd[c][F8 ? 0 : (BLK / 8) * ps];
        if (F8) {
          const float r = s > 0.0f ? as_f((unsigned)(254 - (int)sbc[c]) << 23) : 0.0f;  // 1/s, exact
#pragma unroll
          for (int w = 0; w < BLK / 4; ++w) {
            float q[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_fmed3f(v(4 * w + k) * r, -448.0f, 448.0f);
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
            out[w] = (unsigned)word;
          }
        } else {
          encode_block<BLK>(v, s, FMT == 1, out);
        }
      }
      sbp[ps] = sbc[0] | (sbc[1] << 8);
    }
    // scale bytes of channel d sit at tile offset d*NB + block. NVFP4: this lane has blocks
    // 2j, 2j+1 of both channels; the lane 16 above has 2j+2, 2j+3. MX: blocks j of both
    // channels; lanes 16, 32, 48 above have blocks 1, 2, 3.
    uint8_t* srun = scales + (bh * ntiles + kt) * (int64_t)(D * NB);
    if (NV) {
      const unsigned mine = (sbp[0] & 0xFFu) | ((sbp[1] & 0xFFu) << 8) | ((sbp[0] & 0xFF00u) << 8) | ((sbp[1] & 0xFF00u) << 16);
      const unsigned up = __shfl_down(mine, 16, 64);  // blocks 2j+2, 2j+3 (lanes with j even use it)
      // j even: dword of blocks 4(j/2)..+3 for channel 2dp (lo halves) and 2dp+1 (hi halves)
      const unsigned ch0 = (mine & 0xFFFFu) | (up << 16), ch1 = (mine >> 16) | (up & 0xFFFF0000u);
      // lanes j = 0 and j = 2 swap so that each stores 8 contiguous bytes: j = 0 takes channel
      // 2dp (blocks 0..7), j = 2 channel 2dp+1
      const unsigned give = j == 0 ? ch1 : ch0;
      const unsigned got = __shfl_xor(give, 32, 64);
      if ((j & 1) == 0) {
        const unsigned lo = j == 0 ? ch0 : got, hi = j == 0 ? got : ch1;
        *reinterpret_cast<uint2*>(srun + (2 * dp + (j >> 1)) * NB) = make_uint2(lo, hi);
      }
    } else {
      const unsigned s1 = __shfl_down(sbp[0], 16, 64), s2 = __shfl_down(sbp[0], 32, 64), s3 = __shfl_down(sbp[0], 48, 64);
      if (j == 0) {
        const unsigned lo01 = (sbp[0] & 0xFFu) | ((s1 & 0xFFu) << 8), lo23 = (s2 & 0xFFu) | ((s3 & 0xFFu) << 8);
        const unsigned hi01 = ((sbp[0] >> 8) & 0xFFu) | (s1 & 0xFF00u), hi23 = ((s2 >> 8) & 0xFFu) | (s3 & 0xFF00u);
        *reinterpret_cast<uint2*>(srun + 2 * dp * NB) = make_uint2(lo01 | (lo23 << 16), hi01 | (hi23 << 16));
      }
    }
    if (HAT) {
      // this lane's slots 32j..32j+31 of channels 2dp and 2dp+1: words 2ps, 2ps+1 of channel c
      // belong to block 2j+ps, whose scale byte is byte c of sbp[ps]
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        v8h* dst = reinterpret_cast<v8h*>(vh + ((bh * ntiles + kt) * D + 2 * dp + c) * KV_TILE + 32 * j);
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
          const _Float16 sh = e4m3_to_f16((sbp[ps] >> (8 * c)) & 0xFFu);
          dst[2 * ps] = dequant8(wd[c][2 * ps], v2h{sh, sh});
          dst[2 * ps + 1] = dequant8(wd[c][2 * ps + 1], v2h{sh, sh});
        }
      }
    }
  };
  // Two register buffers: tiles kt0 and kt0+1 are both in flight from the start, and each
  // buffer is refilled two tiles ahead as soon as it is staged.
  uint4 bufa[PPT], bufb[PPT];
  load(kt0, bufa);
  if (kt0 + 1 < kt1) load(kt0 + 1, bufb);
  for (int kp = kt0; kp < kt1; kp += 2) {
    unsigned wd[2][LW];
    step(kp, bufa, kp + 2, wd);
    store_codes(kp, wd);
    if (kp + 1 < kt1) {
      step(kp + 1, bufb, kp + 3, wd);
      store_codes(kp + 1, wd);
    }
  }
}

// tiles per workgroup of the V quantiser: 4 or 2 (whole tile pairs), keeping at least 2048
// workgroups where the shape allows
inline int v_tiles_per_wg(int64_t ntiles, int BH) {
  int tpw = 4;
  while (tpw > 2 && ((ntiles + tpw - 1) / tpw) * BH < 2048) tpw /= 2;
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
  const dim3 grid((unsigned)((nt + tpw - 1) / tpw), (unsigned)BH), block(2 * D);
  if (D == 64) quant_v_tile_kernel<64, 2><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, N, Np, tpw, nullptr);
  else quant_v_tile_kernel<128, 2><<<grid, block, 0, st>>>((const __half*)x, (uint8_t*)codes, (uint8_t*)scales, N, Np, tpw, nullptr);
  return hipGetLastError();
}

// vh: NULL, or (NVFP4 only) where V-hat goes
hipError_t launch_quant_v(bool mx, const void* x, int BH, int N, int D, void* codes, void* scales, void* vh,
                          hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const __half* xp = (const __half*)x;
  uint8_t *c = (uint8_t*)codes, *s = (uint8_t*)scales;
  _Float16* h = (_Float16*)vh;
  const int64_t nt = Np / KV_TILE;
  const int tpw = v_tiles_per_wg(nt, BH);
  const dim3 grid((unsigned)((nt + tpw - 1) / tpw), (unsigned)BH), block(2 * D);
  if (mx) {
    if (D == 64) quant_v_tile_kernel<64, 1><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw, nullptr);
    else quant_v_tile_kernel<128, 1><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw, nullptr);
  } else if (h) {
    if (D == 64) quant_v_tile_kernel<64, 0, true><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw, h);
    else quant_v_tile_kernel<128, 0, true><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw, h);
  } else {
    if (D == 64) quant_v_tile_kernel<64, 0><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw, nullptr);
    else quant_v_tile_kernel<128, 0><<<grid, block, 0, st>>>(xp, c, s, N, Np, tpw, nullptr);
  }
  return hipGetLastError();
}

// NVFP4 K codes and scales with K-hat at kh ([BH][Np][D] fp16)
hipError_t launch_quant_k_hat(const void* x, int BH, int N, int D, void* codes, void* scales, void* kh,
                              hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const dim3 grid((unsigned)((Np * (D / 16) + 255) / 256), (unsigned)BH), block(256);
  const __half* xp = (const __half*)x;
  uint8_t *c = (uint8_t*)codes, *s = (uint8_t*)scales;
  _Float16* h = (_Float16*)kh;
  if (D == 64) quant_k_hat_kernel<64><<<grid, block, 0, st>>>(xp, c, s, N, Np, h);
  else quant_k_hat_kernel<128><<<grid, block, 0, st>>>(xp, c, s, N, Np, h);
  return hipGetLastError();
}

}  // namespace sage
