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
// rne(fl32(x * fl32(127 / a))); the gradient kernels form P's and dS's within an ulp of these
// (recip127, codes16).
//
// CDNA4 design.
//   - prep kernels, one workgroup per (batch*head, 64-token block): NVFP4 Q^ and K^ are
//     dequantised from FP4 to bf16 (exact: a code times its scale has at most 6 significant bits
//     and lies in bf16's exponent range); for MXFP4 Q and K the prep instead lays out their E8M0
//     scales per 64-token block for the FP4 MFMA. Q^, K^ and dO are encoded to INT8 per (channel,
//     block), stored channel-major in the token order below; the dO prep also forms D_i in fp32.
//   - dK/dV kernel, one workgroup of 12 (D = 128) or 16 (D = 64) waves per (batch*head, block of
//     192 or 256 keys): each wave owns 16 keys and keeps their K^ (bf16, or MXFP4 codes) and
//     V (fp16) rows as MFMA B operands in registers while 64-query tiles stream into LDS by
//     asynchronous buffer loads into LDS (buffer_load ... lds), double-buffered, one barrier per
//     tile. S = Q^ K^T and dP = dO V^T take 16x16x32 MFMAs (with MXFP4 Q and K, S takes one
//     block-scaled FP4 16x16x128 MFMA per subtile on the codes themselves); a lane then holds 16
//     (query, key) values of one key, at queries 16s + 4g + i
//     (subtile s, lane group g, element i). P and dS are therefore lane-local, a key's block
//     maximum takes two cross-lane swaps, and a lane's 16 codes are directly the A operand of a
//     16x16x64 INT8 MFMA whose K slots 16g + 4s + i hold those queries; the INT8 dO and Q^ are
//     stored in that slot order. One workgroup per CU (two 49 KB tile buffers at D = 128), three
//     waves per SIMD at D = 128 (at most 168 VGPRs), four at D = 64.
//   - dQ kernel: the mirror image, one wave per 16 queries looping over 64-key tiles. dQ gets
//     a kernel of its own instead of atomic adds, so every result is deterministic.
#include "device.h"

namespace sage {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 f16;

constexpr int BB = 64;                          // token block of the INT8 operands and tile size
constexpr float LOG2E = 1.4426950408889634f;
// lse * log2(e) stored for token positions past N: exp2(x - PAD_L2) is exactly 0 for any finite
// score x, so such a query's P and dS vanish without a per-element mask
constexpr float PAD_L2 = 1.0e30f;

// Token held by slot p of a 64-token block: slot 16g + 4s + i holds token 16s + 4g + i (an
// involution). A wave's 16x16 MFMA results for four 16-token subtiles put token 16s + 4g + i in
// lane group g, subtile s, element i; the 16x16x64 INT8 MFMA reads K slots 16g + [0, 16) from
// lane group g.
__host__ __device__ inline int slot_token64(int p) { return 16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3); }

// fl32(a / b) and fl32(b / a) for the INT8 scale: double division rounded once more to fp32
// equals the correctly rounded fp32 quotient (53 >= 2 * 24 + 2).
__device__ __forceinline__ float div_rn(float a, float b) { return (float)((double)a / (double)b); }

// The scale and reciprocal of a block of P or dS inside the gradient kernels: a * fl32(1/127) and
// 127 * rcp(a) (v_rcp_f32, 1 ulp), 0 for a = 0. They differ from fl32(a / 127) and fl32(127 / a)
// by at most about an ulp, which moves a result far less than its float32 tolerance and a code
// only where x * r lies within a few ulp of a half-integer, where either rounding is allowed.
// The operand preparation uses the exact quotients (its codes are compared bit for bit).
constexpr float INV127 = 1.0f / 127.0f;
__device__ __forceinline__ float recip127(float a) { return a > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(a) : 0.0f; }

// Four integers in [-127, 127] -> one dword, the first in the low byte.
__device__ __forceinline__ int pack4(int a, int b, int c, int d) {
  return (a & 0xFF) | ((b & 0xFF) << 8) | ((c & 0xFF) << 16) | ((d & 0xFF) << 24);
}

// ---------------------------------------------------------------------------------------------
// Prep: one workgroup per (block of 64 tokens, batch*head). SRC 0: NVFP4 codes (also writes the
// bf16 values), 1: MXFP4 codes (also writes the block's E8M0 scale table), 2: fp16 dO (also writes
// D_i from dO and O, and lse * log2 e; both [.., Np], past N 0 and PAD_L2). INT8 scales are
// stored block-major, [.., Np / 64, D].
// ---------------------------------------------------------------------------------------------
template <int D, int SRC>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const f16* __restrict__ x, const f16* __restrict__ o,
                                                       int N, int Np, __bf16* __restrict__ xh,
                                                       uint8_t* __restrict__ tab,
                                                       int8_t* __restrict__ q8, float* __restrict__ q8s,
                                                       const float* __restrict__ lse, float* __restrict__ l2,
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
        if (ch == 0) {
          dl[bh * Np + tok] = dot;
          l2[bh * Np + tok] = lse[row] * LOG2E;
        }
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
        if constexpr (SRC == 0) {
          __bf16* dst = xh + row * D + ch * VPT;
#pragma unroll
          for (int u = 0; u < VPT / 8; ++u) {
            v8bf b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (__bf16)v[8 * u + e];
            *reinterpret_cast<v8bf*>(dst + 8 * u) = b;
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < VPT; ++u) v[u] = 0.0f;
      if constexpr (SRC == 2) {
        if (ch == 0 && tok < Np) {
          dl[bh * Np + tok] = 0.0f;
          l2[bh * Np + tok] = PAD_L2;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) sx[n][ch * VPT + u] = v[u];
  }
  __syncthreads();

  // MXFP4: the E8M0 scales of the block's 64 tokens in the order the gradient kernels read them
  // (mx_tab_index), rows past N repeating row N - 1
  if constexpr (SRC == 1) {
    constexpr int NBD = D / 32;
    if (tid < BB * NBD) {
      const int gg = tid >> 6, cc = (tid >> 2) & 15, ss = tid & 3;
      const int tok = min(blk * BB + 16 * ss + cc, N - 1);
      tab[(bh * nb + blk) * (BB * NBD) + tid] = scales[(bh * N + tok) * NBD + gg];
    }
  }

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
      for (int e = 0; e < 4; ++e) {
        const int* c4 = cq + 16 * u + 4 * e;
        wv[e] = pack4(c4[0], c4[1], c4[2], c4[3]);
      }
      *reinterpret_cast<v4i*>(dst + 16 * u) = wv;
    }
    if (h == 0) q8s[(bh * nb + blk) * D + d] = a > 0.0f ? div_rn(a, 127.0f) : 0.0f;
  }
}

// ---------------------------------------------------------------------------------------------
// Shared pieces of the two gradient kernels.
// ---------------------------------------------------------------------------------------------
// Waves per workgroup, one workgroup per CU (LDS): three per SIMD at D = 128 (at most 168 VGPRs),
// four at D = 64 (at most 128 VGPRs).
template <int D>
constexpr int nwave() { return D == 64 ? 16 : 12; }
template <int D>
constexpr int wblock() { return 16 * nwave<D>(); }  // keys (dK/dV) or queries (dQ) per workgroup

template <int D>
struct BwdTile {
  static constexpr int T16 = BB * 2 * D;  // bytes of a 16-bit tile (64 tokens x D)
  static constexpr int T8 = D * BB;       // bytes of an INT8 tile (D channels x 64 slots)
  static constexpr int W16 = T16 / 1024;  // wave-wide copies (16 bytes per lane) per 16-bit tile
  static constexpr int W8 = T8 / 1024;    // ... per INT8 tile
  static constexpr int KK = D / 32;       // k steps of the 16x16x32 MFMAs
  static constexpr int NN = D / 16;       // 16-channel output subtiles
  static constexpr int T4 = BB * D / 2;   // bytes of an FP4 code tile (64 tokens x D / 2)
  static constexpr int W4 = T4 / 1024;    // ... its wave-wide copies
  static constexpr int TS = BB * D / 32;  // bytes of an MXFP4 scale table (64 tokens x D / 32)
  // The FP4 codes and their table stand in for a 16-bit tile: the table is copied by a whole wave
  // (lanes past TS bytes read zeros into the slack behind it), so the copy needs no lane branch
  static_assert(T4 + 1024 <= T16, "room for a wave-wide copy of the scale table");
};

// LDS tiles carry no padding. An MFMA operand read has 16 lanes fetch one 16-byte chunk from
// each of 16 consecutive rows; storing chunk c of row r at chunk slot c ^ swz(r) gives those 16
// reads 16 different bank groups.
template <int D>
__device__ __forceinline__ int swz16(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
__device__ __forceinline__ int swz8(int d) { return (d >> 2) & 3; }

// Max over the four lanes {l, l^16, l^32, l^48} by fmaxf. The plain-instruction form the forward
// kernels use (xg_max) gives the same values here, but with it the compiler spilled five VGPRs of
// the causal D = 128 dK/dV kernel into scratch, reloaded in every tile.
__device__ __forceinline__ float xg_fmax(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u(v), as_u(v), false, false);
  v = fmaxf(as_f(p[0]), as_f(p[1]));
  auto r = __builtin_amdgcn_permlane32_swap(as_u(v), as_u(v), false, false);
  return fmaxf(as_f(r[0]), as_f(r[1]));
}

// Asynchronous copy of 16 bytes per lane into LDS (buffer_load_dwordx4 ... lds) through a buffer
// resource of `nbytes` bytes at `base`: lane i reads base + voff, or 0 where voff >= nbytes, and
// writes lds + 16 i. base and lds are the same for the whole wave (base in SGPRs, so a lane's
// address is one 32-bit offset); vmcnt counts completion.
// base and nbytes go through readfirstlane: they are uniform, but the compiler may hold a value
// they derive from in VGPRs (N, after a divergent branch of the prologue assigned it on both
// sides), and a buffer resource in VGPRs costs a waterfall loop per copy. readfirstlane returns
// an int: each half is taken back as unsigned before it is widened, so the low half is not
// sign-extended into the high one.
__device__ __forceinline__ void lds_copy16(const void* base, unsigned nbytes, unsigned voff, void* lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
  const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
  const int nu = __builtin_amdgcn_readfirstlane((int)nbytes);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), 0, nu, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Jobs [J0, J1) of a tile's copy schedule, dealt round-robin over NWAVE waves (job j to wave
// j % NWAVE): f(j - J0) for this wave's. Each kind of copy gets a loop of its own, so no two kinds
// share a call site whose buffer resource the compiler would merge into VGPRs.
template <int J0, int J1, int NWAVE, typename F>
__device__ __forceinline__ void wave_jobs(int wave, F f) {
  for (int j = J0 + (wave - J0 % NWAVE + NWAVE) % NWAVE; j < J1; j += NWAVE) f(j - J0);
}

// Copy j of a 16-bit tile: rows [t0, t0 + 64) of one head of a [.., N, D] tensor starting at
// `head` (t0 < N); a row past N reads zeros. Such rows only meet P = 0: queries past N carry the
// lse padding (P underflows to exactly 0) and keys past N are masked.
template <int D>
__device__ __forceinline__ void copy16_job(int j, int lane, const uint8_t* head, int t0, int N, uint8_t* tile) {
  int r, cs;
  if constexpr (D == 128) {
    r = 4 * j + (lane >> 4);
    cs = lane & 15;
  } else {
    r = 8 * j + (lane >> 3);
    cs = lane & 7;
  }
  lds_copy16(head + (int64_t)t0 * (2 * D), (unsigned)(N - t0) * (2 * D), (unsigned)(r * (2 * D) + 16 * (cs ^ swz16<D>(r))),
             tile + 1024 * j);
}

// Copy j of an INT8 tile: 64 slots of every channel, starting at blk0 = codes + (bh D) Np + t0
// (the head's codes end D Np - t0 bytes later).
template <int D>
__device__ __forceinline__ void copy8_job(int j, int lane, const int8_t* blk0, int Np, int t0, uint8_t* tile) {
  const int d = 16 * j + (lane >> 2);
  lds_copy16(blk0, (unsigned)(D * Np - t0), (unsigned)(d * Np + 16 * ((lane & 3) ^ swz8(d))), tile + 1024 * j);
}

// MFMA A operand (8 x 16 bits) of tile row r, channels 32 kk + 8 g .. + 7; sw = swz16(r), which
// for r = 16 s + col equals swz16(col).
template <int D, typename V>
__device__ __forceinline__ V read16(const uint8_t* tile, int r, int kk, int g, int sw) {
  return *reinterpret_cast<const V*>(tile + r * (2 * D) + 16 * ((4 * kk + g) ^ sw));
}
// INT8 MFMA B operand of channel d, slots 16 g .. + 15; sw8 = swz8(d) = swz8(col) for d = 16 n + col.
__device__ __forceinline__ v4i read8(const uint8_t* tile, int d, int g, int sw8) {
  return *reinterpret_cast<const v4i*>(tile + d * BB + 16 * (g ^ sw8));
}

// MXFP4 operands of the S recompute (MXFP4 Q and K): S = Q^ K^T runs on the block-scaled FP4
// MFMA, whose lane (row c, group g) supplies the 32 E2M1 values of K block g of row c (16 bytes)
// and their E8M0 scale. A 64-token tile keeps the codes, D / 2 bytes per row, with chunk c of
// row r at slot c ^ swz4(r), which spreads the 16 rows a lane group reads over distinct bank
// groups. The tile's scales come from the prep's table: byte 4 (16 g + c) + s holds the scale of
// token 16 s + c, block g, so a lane's scales for the four subtiles are one dword, and the
// instruction's op_sel picks byte s.
struct Fp4Ops {
  const uint8_t* qc;  // Q codes [BH, N, D/2] and E8M0 scales [BH, N, D/32]
  const uint8_t* qs;
  const uint8_t* kc;  // K codes and scales
  const uint8_t* ks;
  const uint8_t* qt;  // scale tables of Q and K [BH, Np/64, 64 D/32]
  const uint8_t* kt;
};
template <int D>
__device__ __forceinline__ int swz4(int r) { return D == 128 ? (r >> 2) & 3 : (r >> 3) & 1; }

// Copy j of an FP4 code tile: rows [t0, t0 + 64) of one head of a [.., N, D/2] code array
// (t0 < N); a row past N reads zero codes (and only meets P = 0, as in copy16_job).
template <int D>
__device__ __forceinline__ void copy4_job(int j, int lane, const uint8_t* head, int t0, int N, uint8_t* tile) {
  constexpr int RB = D / 2, CPR = RB / 16, RPJ = 64 / CPR;  // row bytes, chunks per row, rows per copy
  const int r = RPJ * j + lane / CPR, cs = lane % CPR;
  lds_copy16(head + (int64_t)t0 * RB, (unsigned)(N - t0) * RB, (unsigned)(r * RB + 16 * (cs ^ swz4<D>(r))), tile + 1024 * j);
}

// FP4 MFMA A operand: the 16 code bytes of tile row r, K block g. At D = 64 the lane groups
// g = 2, 3 repeat blocks 0, 1; the B operand is zero there, so their products vanish.
template <int D>
__device__ __forceinline__ v8i read4(const uint8_t* tile, int r, int g, int sw4) {
  const v4i u = *reinterpret_cast<const v4i*>(tile + r * (D / 2) + 16 * ((g % (D / 32)) ^ sw4));
  v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
  a[0] = u[0]; a[1] = u[1]; a[2] = u[2]; a[3] = u[3];
  return a;
}

// S subtile s: A = FP4 tile rows with scale byte s of sa, B = the wave's own FP4 rows with scale
// byte 0 of sb (s is a constant after unrolling).
__device__ __forceinline__ v4f mfma_fp4(const v8i& a, const v8i& b, int s, int sa, int sb) {
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  switch (s) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 1, sa, 0, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 2, sa, 0, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 3, sa, 0, sb);
  }
}

// The B operand and scale of row `row` (< N) of an FP4 code array: 16 bytes of block g and its
// E8M0 byte; zero codes (scale 1) for g >= D / 32.
template <int D>
__device__ __forceinline__ void own_fp4(const uint8_t* codes, const uint8_t* scales, int64_t row, int g, v8i& b,
                                        int& sb) {
  b = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  sb = 0x7F;
  if (g < D / 32) {
    const v4i u = *reinterpret_cast<const v4i*>(codes + row * (D / 2) + 16 * g);
    b[0] = u[0]; b[1] = u[1]; b[2] = u[2]; b[3] = u[3];
    sb = scales[row * (D / 32) + g];
  }
}

// Codes of 16 values held by a lane (four subtiles s of four elements i) with a common
// reciprocal scale r; byte 4s + i of the result is the code of value [s][i]. One fma adds
// 1.5 * 2^23 to the exact product x * r, which rounds it to the nearest integer (ties to even)
// in the low mantissa bits; the low byte of the result's bits is the two's complement byte of
// that integer. This is rne(fl32(x * r)) except when x * r lies within half an fp32 ulp of a
// half-integer, where either rounding is within the contract. |x| <= the block maximum a and
// r = recip127(a) (within a few ulp of 127 / a) keep |x * r| below 127.5, so the code lies in
// [-127, 127] without a clamp.
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
// dK and dV: one workgroup of nwave<D>() waves per (batch*head, block of 16 nwave<D>() keys);
// 64-query tiles arrive in LDS through asynchronous copies, double-buffered: tile t + 1 is copied
// while tile t is used.
// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool OUT_F32, bool MXS>
__global__ __launch_bounds__(64 * nwave<D>(), 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ qh, const __bf16* __restrict__ kh, const f16* __restrict__ v,
    const f16* __restrict__ dout, const int8_t* __restrict__ q8, const float* __restrict__ q8s,
    const int8_t* __restrict__ do8, const float* __restrict__ do8s, const float* __restrict__ l2,
    const float* __restrict__ dl, int N, int Np, int BH, float c, void* __restrict__ dk, void* __restrict__ dv,
    Fp4Ops f) {
  using T = BwdTile<D>;
  constexpr int NWAVE = nwave<D>(), WB = wblock<D>();
  // the four fp32 runs (scales of Q8 and dO8, lse*log2e, D) get 1 KB slots each, so a whole wave
  // copies each one (lanes past the run read zeros into its slot) and no copy needs a lane branch
  static_assert(4 * D <= 1024 && 4 * BB <= 1024, "fp32 runs fit their 1 KB slots");
  constexpr int O_DO = T::T16, O_Q8 = 2 * T::T16, O_DO8 = O_Q8 + T::T8, O_QS = O_DO8 + T::T8;
  constexpr int O_DOS = O_QS + 1024, O_L = O_DOS + 1024, O_D = O_L + 1024, BUF = O_D + 1024;
  // copies of the Q tile: bf16 rows, or (MXS) FP4 codes and one copy of the scale table
  constexpr int JQ = MXS ? T::W4 + 1 : T::W16;
  constexpr int NJ = JQ + T::W16 + 2 * T::W8 + 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BUF];

  const int nq = Np / BB;
  const int nkb = (N + WB - 1) / WB;
  const int w = xcd_work(blockIdx.x, BH * nkb);
  // bh and kb are uniform; readfirstlane keeps them in SGPRs (the division runs on the VALU), so
  // the copies' buffer resources built from them need no waterfall loop
  const int64_t bh = __builtin_amdgcn_readfirstlane(w / nkb);
  const int kb = __builtin_amdgcn_readfirstlane(w % nkb);  // causal: the heaviest key blocks first
  // the wave index is uniform across a wave: readfirstlane lets the copy schedule branch on scalars
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 4, col = l & 15;
  const int key = kb * WB + wave * 16 + col;
  const int sw = swz16<D>(col), sw8 = swz8(col), sw4 = swz4<D>(col);

  v8bf kreg[MXS ? 1 : T::KK];
  v8h vreg[T::KK];
  v8i kf = {0, 0, 0, 0, 0, 0, 0, 0};
  int ksc = 0x7F;
  if constexpr (MXS) {
    if (key < N) own_fp4<D>(f.kc + bh * N * (D / 2), f.ks + bh * N * (D / 32), key, g, kf, ksc);
  }
#pragma unroll
  for (int kk = 0; kk < T::KK; ++kk) {
    if (key < N) {
      if constexpr (!MXS) kreg[kk] = *reinterpret_cast<const v8bf*>(kh + (bh * N + key) * D + 32 * kk + 8 * g);
      vreg[kk] = *reinterpret_cast<const v8h*>(v + (bh * N + key) * D + 32 * kk + 8 * g);
    } else {
      if constexpr (!MXS) kreg[kk] = v8bf{};
      vreg[kk] = v8h{};
    }
  }
  v4f accK[T::NN], accV[T::NN];
#pragma unroll
  for (int n = 0; n < T::NN; ++n) accK[n] = accV[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const float cl2e = c * LOG2E;

  // causal: query tiles from the last down to the one holding the block's first key; non-causal:
  // every tile. The workgroups of a head run side by side on one XCD and walk the tiles in the
  // same order (causal blocks all start at the last tile), so each tile comes from HBM once and
  // from that XCD's L2 for the others.
  const int qt0 = CAUSAL ? kb * (WB / BB) : 0, nit = nq - qt0;
  auto tile_of = [&](int it) { return CAUSAL ? nq - 1 - it : it; };
  auto issue = [&](int it, uint8_t* buf) {
    const int qt = tile_of(it), t0 = qt * BB;
    constexpr int J8 = JQ + T::W16, JS = J8 + 2 * T::W8;  // first INT8 job, first fp32-run job
    if constexpr (MXS) {
      wave_jobs<0, T::W4, NWAVE>(wave, [&](int j) { copy4_job<D>(j, l, f.qc + bh * N * (D / 2), t0, N, buf); });
      wave_jobs<T::W4, JQ, NWAVE>(wave, [&](int) { lds_copy16(f.qt + (bh * nq + qt) * T::TS, T::TS, 16 * l, buf + T::T4); });
    } else {
      wave_jobs<0, JQ, NWAVE>(wave, [&](int j) {
        copy16_job<D>(j, l, reinterpret_cast<const uint8_t*>(qh + bh * N * D), t0, N, buf);
      });
    }
    wave_jobs<JQ, J8, NWAVE>(wave, [&](int j) {
      copy16_job<D>(j, l, reinterpret_cast<const uint8_t*>(dout + bh * N * D), t0, N, buf + O_DO);
    });
    wave_jobs<J8, J8 + T::W8, NWAVE>(wave, [&](int j) { copy8_job<D>(j, l, q8 + bh * D * Np + t0, Np, t0, buf + O_Q8); });
    wave_jobs<J8 + T::W8, JS, NWAVE>(wave, [&](int j) { copy8_job<D>(j, l, do8 + bh * D * Np + t0, Np, t0, buf + O_DO8); });
    // the fp32 runs: scales of Q8 and of dO8, lse * log2(e), D
    wave_jobs<JS, JS + 1, NWAVE>(wave, [&](int) { lds_copy16(q8s + (bh * nq + qt) * D, 4 * D, 16 * l, buf + O_QS); });
    wave_jobs<JS + 1, JS + 2, NWAVE>(wave, [&](int) { lds_copy16(do8s + (bh * nq + qt) * D, 4 * D, 16 * l, buf + O_DOS); });
    wave_jobs<JS + 2, JS + 3, NWAVE>(wave, [&](int) { lds_copy16(l2 + bh * Np + t0, 4 * BB, 16 * l, buf + O_L); });
    wave_jobs<JS + 3, NJ, NWAVE>(wave, [&](int) { lds_copy16(dl + bh * Np + t0, 4 * BB, 16 * l, buf + O_D); });
  };

  issue(0, lds[0]);
  for (int it = 0; it < nit; ++it) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile it have landed
    __syncthreads();                // every wave's have, and every wave is done with tile it - 1
    if (it + 1 < nit) issue(it + 1, lds[(it + 1) & 1]);
    const uint8_t* buf = lds[it & 1];
    const int q0 = tile_of(it) * BB;

    float P[4][4], dS[4][4];
    float pmax = 0.0f, smax = 0.0f;
    int qsc = 0;
    if constexpr (MXS) qsc = *reinterpret_cast<const int*>(buf + T::T4 + 4 * (16 * (g % (D / 32)) + col));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4f sc = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (MXS) sc = mfma_fp4(read4<D>(buf, 16 * s + col, g, sw4), kf, s, qsc, ksc);
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        if constexpr (!MXS)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read16<D, v8bf>(buf, 16 * s + col, kk, g, sw), kreg[kk],
                                                       sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_f16(read16<D, v8h>(buf + O_DO, 16 * s + col, kk, g, sw), vreg[kk],
                                                    dp, 0, 0, 0);
      }
      const v4f L4 = *reinterpret_cast<const v4f*>(buf + O_L + 4 * (16 * s + 4 * g));
      const v4f D4 = *reinterpret_cast<const v4f*>(buf + O_D + 4 * (16 * s + 4 * g));
      // queries past N have L = PAD_L2 (P = 0); keys past N only reach their own dK and dV rows,
      // which are not stored: only the causal test remains
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = q0 + 16 * s + 4 * g + i;
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cl2e, -L4[i]));
        const float p = (!CAUSAL || key <= qi) ? e : 0.0f;
        P[s][i] = p;
        dS[s][i] = p * (dp[i] - D4[i]);
        pmax = fmaxf(pmax, p);
        smax = fmaxf(smax, fabsf(dS[s][i]));
      }
    }
    pmax = xg_fmax(pmax);
    smax = xg_fmax(smax);
    const v4i aP = codes16(P, recip127(pmax));
    const v4i aS = codes16(dS, recip127(smax));
    const float sP = pmax * INV127, sS = smax * INV127;
    // the accumulator rows are keys 16 * wave + 4g + i; lane 4g + i holds their scales
    float rP[4], rS[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rP[i] = __shfl(sP, 4 * g + i);
      rS[i] = __shfl(sS, 4 * g + i);
    }
    const float* qs = reinterpret_cast<const float*>(buf + O_QS);
    const float* os = reinterpret_cast<const float*>(buf + O_DOS);
#pragma unroll
    for (int n = 0; n < T::NN; ++n) {
      const v4i rv = __builtin_amdgcn_mfma_i32_16x16x64_i8(aP, read8(buf + O_DO8, 16 * n + col, g, sw8),
                                                           v4i{0, 0, 0, 0}, 0, 0, 0);
      const v4i rk = __builtin_amdgcn_mfma_i32_16x16x64_i8(aS, read8(buf + O_Q8, 16 * n + col, g, sw8),
                                                           v4i{0, 0, 0, 0}, 0, 0, 0);
      const float co = os[16 * n + col], cq = qs[16 * n + col];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accV[n][i] = __builtin_fmaf((float)rv[i], rP[i] * co, accV[n][i]);
        accK[n][i] = __builtin_fmaf((float)rk[i], rS[i] * cq, accK[n][i]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = kb * WB + wave * 16 + 4 * g + i;
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
// dQ: one workgroup of nwave<D>() waves per (batch*head, block of 16 nwave<D>() queries); 64-key
// tiles double-buffered through asynchronous copies as in the dK/dV kernel.
// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool OUT_F32, bool MXS>
__global__ __launch_bounds__(64 * nwave<D>(), 1) void bwd_dq_kernel(
    const __bf16* __restrict__ qh, const __bf16* __restrict__ kh, const f16* __restrict__ v,
    const f16* __restrict__ dout, const int8_t* __restrict__ k8, const float* __restrict__ k8s,
    const float* __restrict__ l2, const float* __restrict__ dl, int N, int Np, int BH, float c,
    void* __restrict__ dq, Fp4Ops f) {
  using T = BwdTile<D>;
  constexpr int NWAVE = nwave<D>(), WB = wblock<D>();
  constexpr int O_V = T::T16, O_K8 = 2 * T::T16, O_KS = O_K8 + T::T8, BUF = O_KS + 1024;  // K8 scales: a 1 KB slot
  constexpr int JK = MXS ? T::W4 + 1 : T::W16;  // copies of the K tile (as in the dK/dV kernel)
  constexpr int NJ = JK + T::W16 + T::W8 + 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BUF];

  const int nk = Np / BB;
  const int nqb = (N + WB - 1) / WB;
  const int w = xcd_work(blockIdx.x, BH * nqb);
  const int64_t bh = __builtin_amdgcn_readfirstlane(w / nqb);  // uniform, kept in SGPRs (dK/dV kernel)
  const int qb = __builtin_amdgcn_readfirstlane(CAUSAL ? nqb - 1 - w % nqb : w % nqb);  // heaviest first
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 4, col = l & 15;
  const int query = qb * WB + wave * 16 + col;
  const int sw = swz16<D>(col), sw8 = swz8(col), sw4 = swz4<D>(col);

  v8bf qreg[MXS ? 1 : T::KK];
  v8h oreg[T::KK];
  v8i qf = {0, 0, 0, 0, 0, 0, 0, 0};
  int qsc = 0x7F;
  float Lq = 0.0f, Dq = 0.0f;
  if constexpr (MXS) {
    if (query < N) own_fp4<D>(f.qc + bh * N * (D / 2), f.qs + bh * N * (D / 32), query, g, qf, qsc);
  }
#pragma unroll
  for (int kk = 0; kk < T::KK; ++kk) {
    if (query < N) {
      if constexpr (!MXS) qreg[kk] = *reinterpret_cast<const v8bf*>(qh + (bh * N + query) * D + 32 * kk + 8 * g);
      oreg[kk] = *reinterpret_cast<const v8h*>(dout + (bh * N + query) * D + 32 * kk + 8 * g);
    } else {
      if constexpr (!MXS) qreg[kk] = v8bf{};
      oreg[kk] = v8h{};
    }
  }
  if (query < N) {
    Lq = l2[bh * Np + query];
    Dq = dl[bh * Np + query];
  }
  // keys visible to this lane's query: kj <= klim. A query past N has zero Q^ and dO rows (so S
  // and dP are 0 and dS is 0) and its dQ row is not stored.
  const int klim = CAUSAL ? min(query, N - 1) : N - 1;
  v4f acc[T::NN];
#pragma unroll
  for (int n = 0; n < T::NN; ++n) acc[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const float cl2e = c * LOG2E;

  // causal: key tiles up to the one holding the block's last query; all blocks walk the tiles
  // in the same order (L2 reuse, as in the dK/dV kernel)
  const int nit = CAUSAL ? min(nk, (qb * WB + WB - 1) / BB + 1) : nk;
  auto tile_of = [&](int it) { return it; };
  auto issue = [&](int it, uint8_t* buf) {
    const int kt = tile_of(it), t0 = kt * BB;
    constexpr int J8 = JK + T::W16;  // first INT8 job
    if constexpr (MXS) {
      wave_jobs<0, T::W4, NWAVE>(wave, [&](int j) { copy4_job<D>(j, l, f.kc + bh * N * (D / 2), t0, N, buf); });
      wave_jobs<T::W4, JK, NWAVE>(wave, [&](int) { lds_copy16(f.kt + (bh * nk + kt) * T::TS, T::TS, 16 * l, buf + T::T4); });
    } else {
      wave_jobs<0, JK, NWAVE>(wave, [&](int j) {
        copy16_job<D>(j, l, reinterpret_cast<const uint8_t*>(kh + bh * N * D), t0, N, buf);
      });
    }
    wave_jobs<JK, J8, NWAVE>(wave, [&](int j) {
      copy16_job<D>(j, l, reinterpret_cast<const uint8_t*>(v + bh * N * D), t0, N, buf + O_V);
    });
    wave_jobs<J8, J8 + T::W8, NWAVE>(wave, [&](int j) { copy8_job<D>(j, l, k8 + bh * D * Np + t0, Np, t0, buf + O_K8); });
    wave_jobs<J8 + T::W8, NJ, NWAVE>(wave, [&](int) { lds_copy16(k8s + (bh * nk + kt) * D, 4 * D, 16 * l, buf + O_KS); });
  };

  issue(0, lds[0]);
  for (int it = 0; it < nit; ++it) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < nit) issue(it + 1, lds[(it + 1) & 1]);
    const uint8_t* buf = lds[it & 1];
    const int k0 = tile_of(it) * BB;
    {
      float dS[4][4];
      float smax = 0.0f;
      int ksc = 0;
      if constexpr (MXS) ksc = *reinterpret_cast<const int*>(buf + T::T4 + 4 * (16 * (g % (D / 32)) + col));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v4f sc = {0.0f, 0.0f, 0.0f, 0.0f}, dp = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (MXS) sc = mfma_fp4(read4<D>(buf, 16 * s + col, g, sw4), qf, s, ksc, qsc);
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
          if constexpr (!MXS)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read16<D, v8bf>(buf, 16 * s + col, kk, g, sw),
                                                         qreg[kk], sc, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_f16(read16<D, v8h>(buf + O_V, 16 * s + col, kk, g, sw), oreg[kk],
                                                      dp, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kj = k0 + 16 * s + 4 * g + i;
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cl2e, -Lq));
          const float p = kj <= klim ? e : 0.0f;
          dS[s][i] = p * (dp[i] - Dq);
          smax = fmaxf(smax, fabsf(dS[s][i]));
        }
      }
      smax = xg_fmax(smax);
      const v4i aS = codes16(dS, recip127(smax));
      const float sS = smax * INV127;
      float rS[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rS[i] = __shfl(sS, 4 * g + i);
      const float* ks = reinterpret_cast<const float*>(buf + O_KS);
#pragma unroll
      for (int n = 0; n < T::NN; ++n) {
        const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(aS, read8(buf + O_K8, 16 * n + col, g, sw8),
                                                            v4i{0, 0, 0, 0}, 0, 0, 0);
        const float ck = ks[16 * n + col];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] = __builtin_fmaf((float)r[i], rS[i] * ck, acc[n][i]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qr = qb * WB + wave * 16 + 4 * g + i;
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
//   Q8, K8, dO8 scales fp32 [BH,nb,D] each | D fp32 [BH,Np] | lse * log2(e) fp32 [BH,Np]
// With MXFP4 Q and K the first two regions start with their E8M0 scale tables instead,
// [BH,nb,D/32,16,4] bytes each (byte [b][g][c][s]: token 64 b + 16 s + c, block g).
struct BwdWs {
  int64_t qh, kh, q8, k8, do8, q8s, k8s, do8s, dl, l2, total;
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
  w.dl = off; off += align256(BH * Np * 4);
  w.l2 = off; off += align256(BH * Np * 4);
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
  float* l2 = reinterpret_cast<float*>(base + L.l2);
  const int Np = (N + BB - 1) / BB * BB, nb = Np / BB;
  const dim3 pg(nb, BH);
  const uint8_t* qcb = reinterpret_cast<const uint8_t*>(qc);
  const uint8_t* qsb = reinterpret_cast<const uint8_t*>(qs);
  const uint8_t* kcb = reinterpret_cast<const uint8_t*>(kc);
  const uint8_t* ksb = reinterpret_cast<const uint8_t*>(ks);
  const f16* vh = reinterpret_cast<const f16*>(v);
  const f16* oh = reinterpret_cast<const f16*>(o);
  const f16* doh = reinterpret_cast<const f16*>(dout);
  // MXFP4 Q and K: the first two regions hold their scale tables instead of bf16 values
  uint8_t* qt = base + L.qh;
  uint8_t* kt = base + L.kh;
  const Fp4Ops f = {qcb, qsb, kcb, ksb, qt, kt};
  if (stages & BWD_PREP) {
    if (mx) {
      bwd_prep_kernel<D, 1><<<pg, 256, 0, st>>>(qcb, qsb, nullptr, nullptr, N, Np, nullptr, qt, q8, q8s, nullptr,
                                                nullptr, nullptr);
      bwd_prep_kernel<D, 1><<<pg, 256, 0, st>>>(kcb, ksb, nullptr, nullptr, N, Np, nullptr, kt, k8, k8s, nullptr,
                                                nullptr, nullptr);
    } else {
      bwd_prep_kernel<D, 0><<<pg, 256, 0, st>>>(qcb, qsb, nullptr, nullptr, N, Np, qh, nullptr, q8, q8s, nullptr,
                                                nullptr, nullptr);
      bwd_prep_kernel<D, 0><<<pg, 256, 0, st>>>(kcb, ksb, nullptr, nullptr, N, Np, kh, nullptr, k8, k8s, nullptr,
                                                nullptr, nullptr);
    }
    bwd_prep_kernel<D, 2><<<pg, 256, 0, st>>>(nullptr, nullptr, doh, oh, N, Np, nullptr, nullptr, do8, do8s, lse,
                                              l2, dl);
  }
  constexpr int WB = wblock<D>();
  const int grid = BH * ((N + WB - 1) / WB);
#define SAGE_BWD_LAUNCH(CZ, F32, MXS)                                                                    \
  do {                                                                                                   \
    if (stages & BWD_DKDV)                                                                               \
      bwd_dkdv_kernel<D, CZ, F32, MXS><<<grid, 64 * nwave<D>(), 0, st>>>(qh, kh, vh, doh, q8, q8s, do8, do8s, l2, \
                                                                         dl, N, Np, BH, c, dk, dv, f);   \
    if (stages & BWD_DQ)                                                                                 \
      bwd_dq_kernel<D, CZ, F32, MXS><<<grid, 64 * nwave<D>(), 0, st>>>(qh, kh, vh, doh, k8, k8s, l2, dl, N, Np, \
                                                                       BH, c, dq, f);                    \
  } while (0)
#define SAGE_BWD_FMT(CZ, F32)               \
  do {                                      \
    if (mx) SAGE_BWD_LAUNCH(CZ, F32, true); \
    else SAGE_BWD_LAUNCH(CZ, F32, false);   \
  } while (0)
  if (causal) {
    if (out_f32) SAGE_BWD_FMT(true, true);
    else SAGE_BWD_FMT(true, false);
  } else {
    if (out_f32) SAGE_BWD_FMT(false, true);
    else SAGE_BWD_FMT(false, false);
  }
#undef SAGE_BWD_FMT
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
    return launch_bwd_d<64>(stages, mx, qc, qs, kc, ks, v, o, dout, lse, BH, N, causal, c, dq, dk, dv, out_f32, ws,
                            st);
  return launch_bwd_d<128>(stages, mx, qc, qs, kc, ks, v, o, dout, lse, BH, N, causal, c, dq, dk, dv, out_f32, ws,
                           st);
}

}  // namespace sage
