// attn_mxfp4.hip — fused MXFP4 attention forward for gfx950 on the block-scaled FP4 MFMA.
//
// SageAttention3 (arXiv 2505.11594), DeepTech article, section on FP4 data types: MXFP4 is E2M1
// with one E8M0 scale per 32 values; the pages compare it with NVFP4 for attention. The CDNA4
// instruction v_mfma_scale_f32_16x16x128_f8f6f4 consumes exactly this format: each lane supplies
// 32 consecutive E2M1 values of one row plus their E8M0 scale, so S = Q K^T and P V run natively
// at the FP4 rate with FP32 accumulation.
//
// Schedule: 8 (D = 64: 4) waves x 16 queries per workgroup, 128-key tiles of FP4 codes and
// scales staged in LDS (no dequantisation), S^T = K Q^T so that a lane's 32 scores of one query
// are one MXFP4 block of P in slot order, accumulator kept relative to the current tile maximum.
// At most 128 VGPRs, so four waves share a SIMD. The softmax's VALU work dominates the time:
// on gfx950 MFMA and plain VALU instructions do not overlap (measured), so what counts is the
// number of VALU instructions per score, which the layout keeps at about six. Workgroups are
// ordered so that each XCD walks through whole heads. The next tile's codes stream straight into
// a second set of LDS buffers (buffer loads into LDS) during the whole current tile, with one
// barrier per tile; its scale bytes come through registers. Scale bytes sit in LDS so that a
// lane reads its eight K (or V) scales of a tile as one 8-byte word; the instruction's op_sel
// bits pick the byte.
// Instances: plain MXFP4, Direct-P (normaliser from the rounded P) and FP8-PV (P, V in MXFP8).
// P has no first level (E8M0 scales cover its range): its codes are E = 2^(x - t) quantised with
// the lane-local block's power-of-two scale.
//
// Exactness of the tile maximum: E = 1 exactly for the maximal score, and that value sits on an
// E8M0 scale boundary. E is evaluated as clamp01(exp2(S*k2 - T)) with one fma, where T is the
// tile maximum in log2 units rounded toward -infinity: for the maximal score the fma's exact
// argument is in [0, ulp), so exp2 gives >= 1 and the clamp (folded into v_exp_f32) returns 1.
#include "device.h"

namespace sage {

// waves per workgroup (16 queries each): 8 at D = 128; at D = 64, where a tile's staging is half
// as large, 4 waves (four workgroups per CU) measured faster
template <int D> constexpr int mx_waves() { return D == 64 ? 4 : 8; }

__device__ __forceinline__ unsigned pack_e4(const float* v, float scale) {
  // every byte of w is written below, so its initial value is irrelevant (no register zeroing)
  unsigned w = as_u(v[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
  return w;
}

// Block-scaled MFMA (operand format F: 4 = FP4 E2M1, 0 = FP8 E4M3, the same for A and B) whose A
// scale is byte `sel` of `sa` (the instruction's op_sel bits pick the byte; `sel` is a constant
// after unrolling, so the switch folds away).
template <int F>
__device__ __forceinline__ v4f mfma_sel(const v8i& a, const v8i& b, const v4f& c, int sel, int sa, int sb) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F, F, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F, F, 1, sa, 0, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F, F, 2, sa, 0, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F, F, 3, sa, 0, sb);
  }
}

// Four FP32 values -> four E4M3 bytes of v / 2^floor(log2 scale), round to nearest even (the
// callers keep every quotient within +-448).
__device__ __forceinline__ unsigned pack_e4m3(float v0, float v1, float v2, float v3, float scale) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, v0, v1, scale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, v2, v3, scale, true);
  return (unsigned)(unsigned short)w[0] | ((unsigned)(unsigned short)w[1] << 16);
}

__device__ __forceinline__ float exp2_01(float x) {
  return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x), 0.0f, 1.0f);
}

// PV8: P and V in MXFP8 (E4M3 elements, E8M0 scale per 32 slots) instead of MXFP4; the PV
// products then run at the FP8 rate. DIRECT_P (MXFP4 only): the normaliser sums the rounded P.
//
// FP8 operand layout (measured on gfx950): in v_mfma_scale_f32_16x16x128_f8f6f4 with FP8
// operands, lane group g (lanes 16g .. 16g+15) holds K-indices 16g .. 16g+15 in its first four
// VGPRs and 64+16g .. 64+16g+15 in the last four, while the scale of K-block b (indices 32b ..
// 32b+31) still comes from lane group b. So a lane's 32 P values are not one block: its first
// half shares block g/2 with the partner group g^1, its second half block 2 + g/2. To make the
// S^T layout deliver exactly those slots, the PV8 instance stores the K tile in LDS under a
// row permutation rho (a bit permutation of the key index) and reads subtile rows as before:
// lane group g of subtile t then holds slots 16g + 4t + i (t < 4) and 64 + 16g + 4(t-4) + i
// (t >= 4), i.e. P's B-operand bytes in place, and the block maxima need one exchange with
// the partner group.
__host__ __device__ constexpr int pv8_rho(int key) {
  return (key & 0x33) | (((key >> 3) & 1) << 6) | (((key >> 2) & 1) << 3) | (((key >> 6) & 1) << 2);
}

// inverse of pv8_rho: rho moves key bit 6 to 2, 2 to 3 and 3 to 6
__host__ __device__ constexpr int pv8_rho_inv(int row) {
  return (row & 0x33) | (((row >> 2) & 1) << 6) | (((row >> 3) & 1) << 2) | (((row >> 6) & 1) << 3);
}

// Asynchronous copy of 16 bytes per lane into LDS through a buffer resource of `nbytes` bytes
// at `base` (wave-uniform): lane i reads base + voff, or 0 where voff >= nbytes, and writes
// lds + 16 i; vmcnt counts completion.
__device__ __forceinline__ void lds_copy16(const void* base, unsigned nbytes, unsigned voff, void* lds) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// One byte per lane through a buffer resource of `nbytes` bytes at `base` (wave-uniform): lane i
// reads base + voff, or 0 where voff >= nbytes. With the tile's base in the resource the lane's
// offset stays the same from tile to tile, so no address arithmetic is repeated per tile.
__device__ __forceinline__ unsigned load_byte(const void* base, unsigned nbytes, unsigned voff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, 0, 0);
}

// The lane's partner value after a permlane swap of `mine` (the pair holds both, in an order
// that depends on the lane; equal values make either choice right).
__device__ __forceinline__ unsigned partner_of(unsigned mine, unsigned p0, unsigned p1) {
  return p0 == mine ? p1 : p0;
}
template <int D, bool CAUSAL, bool OUT_F32, bool DIRECT_P, bool PV8>
__global__ __launch_bounds__(64 * mx_waves<D>(), 4) void attn_mxfp4_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
    int N, int64_t Np, int nqt, int nwork, int cgroup, float k2, void* __restrict__ out,
    float* __restrict__ lse) {
  static_assert(!(PV8 && DIRECT_P), "Direct-P is defined for MXFP4 P");
  constexpr int MX_NT = 64 * mx_waves<D>(), MX_BQ = 16 * mx_waves<D>();
  constexpr int NW = mx_waves<D>();       // waves per workgroup
  constexpr int VB = PV8 ? 128 : 64;      // V code bytes per channel and tile (128 slots)
  constexpr int NBD = D / 32;             // MXFP4 blocks along D (16-byte chunks per K row)
  // LDS tiles of the codes: dense rows (K: D/2 bytes per key, V: VB bytes per channel), so that
  // one copy instruction of a wave fills 1 KB; chunk q of row r sits at slot q ^ swz(r), so that
  // the 16 rows a lane group reads hit distinct bank groups. Two sets of buffers: tile kt is read
  // from set kt mod 2 while tile kt + 1 streams into the other.
  constexpr int KT_BYTES = KV_TILE * (D / 2), VT_BYTES = D * VB;
  static_assert(KT_BYTES % 1024 == 0 && VT_BYTES % 1024 == 0, "whole 1 KB copies");
  __shared__ __attribute__((aligned(16))) uint8_t sKc0[KT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sKc1[KT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sVc0[VT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sVc1[VT_BYTES];
  // scale bytes, laid out so that lane (g, c) finds its eight per tile in one 8-byte word:
  // K: byte (4c + g) * 8 + t holds key 16t + c's block g; V: byte (4c + g) * 8 + dt holds
  // channel 16dt + c's block g (dt < D/16)
  __shared__ __attribute__((aligned(16))) uint8_t sKs0[KV_TILE * 4];
  __shared__ __attribute__((aligned(16))) uint8_t sKs1[KV_TILE * 4];
  __shared__ __attribute__((aligned(16))) uint8_t sVs0[16 * 4 * 8];
  __shared__ __attribute__((aligned(16))) uint8_t sVs1[16 * 4 * 8];
  auto kswz = [](int r) { return D == 128 ? (r >> 1) & 3 : (r >> 2) & 1; };
  auto vswz = [](int r) { return PV8 ? (r & 7) : (r >> 1) & 3; };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int work = xcd_work((int)blockIdx.x, nwork);
  int64_t bh = work / nqt;
  int qt = work % nqt;
  if (CAUSAL) causal_work(work, nqt, nwork / nqt, cgroup, bh, qt);
  const int q0 = qt * MX_BQ;
  const int qi = q0 + 16 * w + c;

  // Q operand: lane holds the 32 codes of block g of query qi (zeros past D) and its scale.
  v8i qf = {0, 0, 0, 0, 0, 0, 0, 0};
  int qsc = 127;
  if (qi < N && g < NBD) {
    const int64_t row = bh * N + qi;
    const uint4 u = *reinterpret_cast<const uint4*>(qc + row * (D / 2) + 16 * g);
    qf[0] = (int)u.x; qf[1] = (int)u.y; qf[2] = (int)u.z; qf[3] = (int)u.w;
    qsc = qs[row * NBD + g];
  }

  float m_u = -INFINITY, R = -INFINITY, l = 0.0f;
  v4f Lacc = {0, 0, 0, 0};  // Direct-P: every element holds the running sum of P-hat of query qi
  v4f O[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) O[dt] = v4f{0, 0, 0, 0};

  const int ntiles = (int)(Np / KV_TILE);
  const int kt_end = CAUSAL ? min(ntiles, (q0 + MX_BQ - 1) / KV_TILE + 1) : ntiles;

  // Staging: the next tile's codes are copied straight into the other LDS set (buffer loads into
  // LDS, issued right after the current tile's barrier), so they stream in during the whole
  // tile; its scale bytes come into registers with them and are written at the top of the next
  // tile. One barrier per tile: set kt mod 2 was last read in tile kt - 2, before the barrier of
  // tile kt - 1. Copy job j fills bytes [1024 j, +1024) of a tile; lane l takes the global chunk
  // that belongs at its slot, so a lane's source offsets are the same from tile to tile. Key rows
  // past N lie outside the copy's buffer range and read as zero codes (their scores are masked).
  static_assert(MX_NT == KV_TILE * NBD && MX_NT == 4 * D, "one K and one V scale byte per thread and tile");
  constexpr int KJOBS = KT_BYTES / 1024, VJOBS = VT_BYTES / 1024;
  constexpr int KPW = (KJOBS + NW - 1) / NW, VPW = (VJOBS + NW - 1) / NW;  // copies per wave
  const uint8_t* kc_h = kc + bh * N * (D / 2);
  const uint8_t* ks_h = ks + bh * N * NBD;
  // V codes and scales are stored tile by tile ([Np/128][D][VB] and [Np/128][D][4]): a tile's
  // codes are one contiguous run of D*VB bytes, its scales one of 4*D bytes, byte tid of which is
  // channel tid/4, block tid%4
  const uint8_t* vc_h = vc + bh * D * (PV8 ? Np : Np / 2);
  const uint8_t* vs_h = vs + bh * D * (Np / 32);
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, known to be uniform
  unsigned koff[KPW], voff[VPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int q = 64 * (NW * i + w) + lane, r = q / NBD, cs = q % NBD;  // LDS row and slot
    koff[i] = (unsigned)((PV8 ? pv8_rho_inv(r) : r) * (D / 2) + 16 * (cs ^ kswz(r)));
  }
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int q = 64 * (NW * i + w) + lane, r = q / (VB / 16), cs = q % (VB / 16);
    voff[i] = (unsigned)(r * VB + 16 * (cs ^ vswz(r)));
  }
  unsigned rks = 0, rvs = 0;
  auto issue = [&](int kt, uint8_t* sKc, uint8_t* sVc) {
    const uint8_t* kb = kc_h + (int64_t)kt * KV_TILE * (D / 2);
    const unsigned kn = (unsigned)(min(N - kt * KV_TILE, KV_TILE) * (D / 2));
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int job = NW * i + wu;
      if (job < KJOBS) lds_copy16(kb, kn, koff[i], sKc + 1024 * job);
    }
    const uint8_t* vb = vc_h + (int64_t)kt * (VB * D);
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int job = NW * i + wu;
      if (job < VJOBS) lds_copy16(vb, (unsigned)(VB * D), voff[i], sVc + 1024 * job);
    }
    // this thread's scale bytes: K key kt*128 + tid/NBD, block tid%NBD (keys past N read 0, the
    // E8M0 value 2^-127, times their zero codes: an exact 0 score, masked anyway); V byte tid
    rks = load_byte(ks_h + (int64_t)kt * KV_TILE * NBD, kn / (D / 2) * NBD, (unsigned)tid);
    rvs = load_byte(vs_h + (int64_t)kt * (4 * D), (unsigned)(4 * D), (unsigned)tid);
  };
  // Direct-P: a 16 x 128 tile of ones (E2M1 code 2 = 1.0 in every nibble), the A operand of the
  // normaliser's MFMA. The empty asm makes its value opaque, so it stays in four VGPRs for the
  // whole loop instead of being rebuilt from a constant in every tile.
  unsigned one0 = 0x22222222u, one1 = one0, one2 = one0, one3 = one0;
  if (DIRECT_P) asm volatile("" : "+v"(one0), "+v"(one1), "+v"(one2), "+v"(one3));
  // One key tile, from LDS set (sKc, sKs, sVc, sVs), copying the next one into (nKc, nVc). The
  // sets are __restrict__ parameters: the compiler then knows that the copies and this tile's
  // reads touch different memory, and puts no wait for the copies before the reads.
  auto tile = [&](int kt, uint8_t* __restrict__ sKc, uint8_t* __restrict__ sKs, uint8_t* __restrict__ sVc,
                  uint8_t* __restrict__ sVs, uint8_t* __restrict__ nKc, uint8_t* __restrict__ nVc) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies and scale loads of tile kt have landed
    {
      const int r = PV8 ? pv8_rho(tid / NBD) : tid / NBD;  // LDS row of this thread's key
      sKs[((r & 15) * 4 + tid % NBD) * 8 + (r >> 4)] = (uint8_t)rks;
      const int d = tid >> 2;  // channel d's block tid & 3
      sVs[((d & 15) * 4 + (tid & 3)) * 8 + (d >> 4)] = (uint8_t)rvs;
    }
    __syncthreads();  // every wave's copies of tile kt have landed; every wave is done with kt - 1
    if (kt + 1 < kt_end) issue(kt + 1, nKc, nVc);

    // ---- S^T = K Q^T: one scaled FP4 MFMA per 16-key subtile (K dimension 128 >= D)
    v4f S[8];
    uint2 ksw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (g < NBD) ksw = *reinterpret_cast<const uint2*>(sKs + (c * 4 + g) * 8);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
      if (g < NBD) {
        const int r = 16 * t + c;
        const uint4 u = *reinterpret_cast<const uint4*>(sKc + r * (D / 2) + 16 * (g ^ kswz(r)));
        a[0] = (int)u.x; a[1] = (int)u.y; a[2] = (int)u.z; a[3] = (int)u.w;
      }
      // the scale operand's byte t & 3 is selected by the instruction's op_sel bits
      S[t] = mfma_sel<4>(a, qf, v4f{0, 0, 0, 0}, t & 3, (int)(t < 4 ? ksw.x : ksw.y), qsc);
    }
    const int kbase = kt * KV_TILE;
    if (kbase + KV_TILE > N || (CAUSAL && kbase + KV_TILE - 1 > q0)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kbase + (PV8 ? 64 * (g & 1) + 16 * (t & 3) + 8 * (t >> 2) + 4 * (g >> 1) + i
                                     : 16 * t + 4 * g + i);
          if (j >= N || (CAUSAL && j > qi)) S[t][i] = -INFINITY;
        }
        // the masked scores leave the branch as they are (an empty asm that "modifies" them): the
        // compiler would otherwise move the selects after the branch, into every tile's path
        asm volatile("" : "+v"(S[t]));
      }
    }
    // ---- online softmax in log2 units
    // bmx: the maximum of S over the lane's P block (PV8: over the block of its first half,
    // which it shares with the partner group g^1; bmB: the same for the second half)
    float bmx = -INFINITY, bmB = -INFINITY, tS;
    if (PV8) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bmx = max3f(bmx, fmaxf(S[t][0], S[t][1]), fmaxf(S[t][2], S[t][3]));
        bmB = max3f(bmB, fmaxf(S[t + 4][0], S[t + 4][1]), fmaxf(S[t + 4][2], S[t + 4][3]));
      }
      bmx = pair16_max(bmx);
      bmB = pair16_max(bmB);
      tS = pair32_max(fmaxf(bmx, bmB));
    } else {
#pragma unroll
      for (int t = 0; t < 8; t += 2) {  // three-input maxima: 16 instructions for 32 values
        bmx = max3f(bmx, max3f(S[t][0], S[t][1], S[t][2]), max3f(S[t][3], S[t + 1][0], S[t + 1][1]));
        bmx = max3f(bmx, S[t + 1][2], S[t + 1][3]);
      }
      tS = xg_max(bmx);
    }
    const bool vis = tS > -INFINITY;
    // tile maximum in log2 units, rounded toward -infinity: when the product was rounded up, step
    // one ulp down, i.e. subtract 1 from the bit pattern of a positive T0 and add 1 to that of a
    // negative one (-0 gives -2^-149; +0 is exact whenever the residual is negative, since k2 > 0).
    // Integer arithmetic and one select, no branches; an empty tile gives T = 0 and is not accepted.
    const float T0 = tS * k2;
    const float Tdn = as_f(as_u(T0) - (unsigned)((__float_as_int(T0) >> 31) | 1));
    float T = __builtin_fmaf(tS, k2, -T0) < 0.0f ? Tdn : T0;
    T = vis ? T : 0.0f;
    const float m_new = fmaxf(m_u, T);
    const bool accept = vis && (T >= m_new - 64.0f);

    // the lane's block: E8M0 scale 2^(floor(log2 amax) - EMAX), amax = the block maximum of E
    // (EMAX = 2 for E2M1, 8 for E4M3); then E chunk by chunk, summed and packed at once. A block
    // that is dropped (its tile rejected, or its amax below the E8M0 range) keeps its codes but
    // takes the scale byte 0, i.e. 2^-127. Once a tile is accepted the normaliser is at least 1
    // in the accumulator's frame (its maximal score has E = 1), and such a block adds at most
    // 2^-127 * 448 * 32 times the largest V value to O, far below FP32 resolution; in exchange the
    // codes need no select or branch.
    constexpr int EMAX = PV8 ? 8 : 2;
    constexpr float AMIN = PV8 ? 0x1p-118f : 0x1p-124f;  // below: X < -126, the block is dropped
    const float amax = exp2_01(__builtin_fmaf(bmx, k2, -T));
    const int X = (int)((as_u(amax) >> 23) & 0xFF) - 127 - EMAX;  // amax is 0 or normal here
    const bool keep = accept && amax >= AMIN;
    const float sc = as_f((unsigned)max(X + 127, 1) << 23);
    float esum = 0.0f;
    v8i pf = {0, 0, 0, 0, 0, 0, 0, 0};
    int psc;
    if (PV8) {
      const float amaxB = exp2_01(__builtin_fmaf(bmB, k2, -T));
      const int XB = (int)((as_u(amaxB) >> 23) & 0xFF) - 127 - EMAX;
      const bool keepB = accept && amaxB >= AMIN;
      const float scB = as_f((unsigned)max(XB + 127, 1) << 23);
      // E4M3 saturates at 448: quotients E / 2^X in [448, 512) clamp to 448
      const float cap = 448.0f * sc, capB = 448.0f * scB;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        float E[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          E[i] = exp2_01(__builtin_fmaf(S[wd][i], k2, -T));
          esum += E[i];
          E[i] = fminf(E[i], wd < 4 ? cap : capB);
        }
        pf[wd] = (int)pack_e4m3(E[0], E[1], E[2], E[3], wd < 4 ? sc : scB);
      }
      // the B operand's scale of K-block g: block 0 (1) is the first half of groups 0, 1 (2, 3),
      // block 2 (3) the second half; groups 1 and 2 take it from their partner across 32 lanes
      const int sA = keep ? X + 127 : 0, sB = keepB ? XB + 127 : 0;
      const unsigned send = (unsigned)(g < 2 ? sB : sA);
      const auto pr = __builtin_amdgcn_permlane32_swap(send, send, false, false);
      const int recv = (int)partner_of(send, pr[0], pr[1]);
      psc = g == 0 ? sA : (g == 3 ? sB : recv);
    } else {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float E[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          E[e] = exp2_01(__builtin_fmaf(S[2 * wd + (e >> 2)][e & 3], k2, -T));
          if (!DIRECT_P) esum += E[e];
        }
        pf[wd] = (int)pack_e4(E, sc);
      }
      psc = keep ? X + 127 : 0;
    }
    if (!accept) esum = 0.0f;
    const float factor = accept ? __builtin_amdgcn_exp2f(R - T) : 1.0f;
    R = accept ? T : R;
    m_u = m_new;
    if (DIRECT_P) Lacc[0] *= factor;  // only element 0 is read
    else l = l * factor + esum;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[dt] *= factor;

    // ---- O^T += V^T P^T: one scaled FP4 (FP8) MFMA per 16 channels; lane group g supplies
    // slots 32g .. 32g+31 (FP8: 16g .. 16g+15 and 64+16g .. 64+16g+15) of V's row 16dt + c and
    // of P's column qi
    uint2 vsw;
    if (D == 128) vsw = *reinterpret_cast<const uint2*>(sVs + (c * 4 + g) * 8);
    else vsw = make_uint2(*reinterpret_cast<const unsigned*>(sVs + (c * 4 + g) * 8), 0u);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      if (PV8) {
        const int r = 16 * dt + c;
        const uint4 u0 = *reinterpret_cast<const uint4*>(sVc + r * VB + 16 * (g ^ vswz(r)));
        const uint4 u1 = *reinterpret_cast<const uint4*>(sVc + r * VB + 16 * ((4 + g) ^ vswz(r)));
        const v8i a = {(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        O[dt] = mfma_sel<0>(a, pf, O[dt], dt & 3, (int)(dt < 4 ? vsw.x : vsw.y), psc);
      } else {
        const int r = 16 * dt + c;
        const uint4 u = *reinterpret_cast<const uint4*>(sVc + r * VB + 16 * (g ^ vswz(r)));
        const v8i a = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        O[dt] = mfma_sel<4>(a, pf, O[dt], dt & 3, (int)(dt < 4 ? vsw.x : vsw.y), psc);
      }
    }
    if (DIRECT_P) {
      // Direct-P normaliser: the sum of the rounded P values, as one more MFMA of P against a
      // 16 x 128 tile of ones (E2M1 code 2 = 1.0, unit scale); all 16 rows of the product equal
      // the row sum, and C's layout hands each lane the sum of its own query qi.
      const v8i ones = {(int)one0, (int)one1, (int)one2, (int)one3, 0, 0, 0, 0};
      Lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf, Lacc, 4, 4, 0, 127, 0, psc);
    }
  };
  issue(0, sKc0, sVc0);
  for (int kt = 0; kt < kt_end; ++kt) {
    const bool odd = kt & 1;
    tile(kt, odd ? sKc1 : sKc0, odd ? sKs1 : sKs0, odd ? sVc1 : sVc0, odd ? sVs1 : sVs0, odd ? sKc0 : sKc1,
         odd ? sVc0 : sVc1);
  }

  const float L = DIRECT_P ? Lacc[0] : xg_sum(l);
  if (qi < N) {
    const float inv = 1.0f / L;
    const int64_t row = bh * N + qi;
    // the row's log-sum-exp (Direct-P: of the rounded P), ln(2^R * L): L sums E in R's frame
    if (lse && g == 0) lse[row] = (R + __builtin_amdgcn_logf(L)) * 0.6931471805599453f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const v4f o = O[dt] * inv;
      if (OUT_F32) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + row * D + 16 * dt + 4 * g) = o;
      } else {
        typedef _Float16 v4h __attribute__((ext_vector_type(4)));
        *reinterpret_cast<v4h*>(reinterpret_cast<_Float16*>(out) + row * D + 16 * dt + 4 * g) =
            v4h{(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
      }
    }
  }
}

template <int D, bool CAUSAL, bool F32, bool DP, bool PV8>
static void launch_mx(const void* const* p, int BH, int N, float k2, void* out, float* lse, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  constexpr int BQ = 16 * mx_waves<D>();
  const int nqt = (N + BQ - 1) / BQ;
  // K and V bytes per head: FP4 codes + E8M0 scales (FP8-PV: V codes are a byte each)
  const int cgroup = causal_group(BH, Np * D * (PV8 ? 3 : 2) / 2 + Np * D / 16);
  attn_mxfp4_kernel<D, CAUSAL, F32, DP, PV8><<<dim3(nqt * BH), dim3(64 * mx_waves<D>()), 0, st>>>(
      (const uint8_t*)p[0], (const uint8_t*)p[1], (const uint8_t*)p[2], (const uint8_t*)p[3],
      (const uint8_t*)p[4], (const uint8_t*)p[5], N, Np, nqt, nqt * BH, cgroup, k2, out, lse);
}

template <bool DP, bool PV8>
static hipError_t launch_mx_any(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                                void* out, bool out_f32, float* lse, hipStream_t st) {
  const float k2 = sm_scale * 1.4426950408889634f;
#define SAGE_MX_CASE(DD, CC, FF) \
  if (D == DD && causal == CC && out_f32 == FF) launch_mx<DD, CC, FF, DP, PV8>(ptrs, BH, N, k2, out, lse, st);
  SAGE_MX_CASE(64, false, false) SAGE_MX_CASE(64, false, true) SAGE_MX_CASE(64, true, false)
  SAGE_MX_CASE(64, true, true) SAGE_MX_CASE(128, false, false) SAGE_MX_CASE(128, false, true)
  SAGE_MX_CASE(128, true, false) SAGE_MX_CASE(128, true, true)
#undef SAGE_MX_CASE
  return hipGetLastError();
}

hipError_t launch_attn_mxfp4(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                             void* out, bool out_f32, float* lse, hipStream_t st) {
  return launch_mx_any<false, false>(ptrs, BH, N, D, causal, sm_scale, out, out_f32, lse, st);
}

hipError_t launch_attn_mxfp4_direct_p(const void* const* ptrs, int BH, int N, int D, bool causal,
                                      float sm_scale, void* out, bool out_f32, float* lse, hipStream_t st) {
  return launch_mx_any<true, false>(ptrs, BH, N, D, causal, sm_scale, out, out_f32, lse, st);
}

hipError_t launch_attn_mx4_pv8(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                               void* out, bool out_f32, float* lse, hipStream_t st) {
  return launch_mx_any<false, true>(ptrs, BH, N, D, causal, sm_scale, out, out_f32, lse, st);
}

}  // namespace sage
