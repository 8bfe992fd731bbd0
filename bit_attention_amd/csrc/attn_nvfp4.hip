// attn_nvfp4.hip — fused NVFP4 attention forward for gfx950.
//
// SageAttention3 (arXiv 2505.11594), DeepTech article: S = Q K^T and P V take FP4 operands in
// 1x16 microscaling blocks (section on the two FP4 obstacles); P is quantised in two levels, each
// token's values first scaled into [0, 448*6], then 1x16 FP4 with E4M3 scales (same section);
// the quantisation of P is fused into the online softmax, whose row-maximum pass also yields the
// block maxima (section on FP4 inference and its hardware implementation); FP32 accumulation.
//
// CDNA4 design. The scaled FP4 MFMA takes only power-of-two (E8M0) block scales, and an E2M1
// code times an E4M3 scale needs up to 6 significant bits, which no FP8/FP6 operand holds. So
// NVFP4 operands are dequantised exactly to fp16 (the code value by the hardware conversion,
// times the E4M3 scale by one fp16 multiply: at most 6 significant bits, 2^-10 .. 2688) and both
// products run on v_mfma_f32_16x16x32_f16.
//   - workgroup = 4 waves = 128 queries of one (batch, head); each wave owns 32 queries as two
//     16-query groups, so every K/V operand read from LDS feeds two MFMAs. Two workgroups fit on
//     a CU (LDS 2 x 64 KB at D = 128, at most 256 VGPRs per wave), so one stages while the other
//     computes.
//   - key tiles of 128: K and V codes of the next tile are loaded into registers while the
//     current tile is computed, then dequantised into LDS between two barriers.
//   - MFMA operands are read from LDS two MFMA pairs ahead through a ring of three fragments
//     (a scheduling barrier per step stops the compiler from hoisting further, which would
//     cost registers: the kernel sits close to the 256-VGPR limit of two waves per SIMD).
//   - each group computes S^T = K Q^T for its 16 queries: after 8 subtiles a lane holds the 32
//     scores of one query at keys 16t + 4g + i, exactly the slot order the quantisation kernel
//     stores V in, so P's 1x16 blocks are lane-local (two per lane per tile), their maxima come
//     out of the row-max pass, and the quantised P is already the B operand of O^T = V^T P^T.
//   - the row max needs two cross-lane swaps (permlane16/32); everything else is lane-local.
//   - accumulator reference: O and l are kept relative to the current tile's maximum, so the
//     MFMA accumulates P2-hat * V-hat directly; one multiply rescales them per tile. A tile whose
//     weight relative to the running maximum is below 2^-64 (its maximum more than 64 below it
//     in log2 units) is dropped for that row.
//   - workgroups are ordered so that each XCD walks through whole heads (K/V stay in its L2).
//   - KV16 instance: K-hat and V-hat come already dequantised to fp16 (kv16_prep_kernel, once per
//     tensor instead of once per query tile) and are copied straight into the swizzled LDS tiles
//     by buffer loads into LDS (no staging registers, no dequantisation in the loop): K tile
//     kt + 1 is copied during the PV products of tile kt, V tile kt during its QK products and
//     softmax. Same arithmetic, same results bit for bit.
#include "device.h"

namespace sage {

constexpr int NV_WAVES = 4;
constexpr int NV_BQ = 32 * NV_WAVES;  // queries per workgroup
constexpr float LOG2_2688 = 11.392317422778762f;  // log2(448 * 6)

// Four E4M3 scale bytes (one dword) -> fp16 values, exact (E4M3 fits fp16).
__device__ __forceinline__ void scales4(unsigned sw, _Float16* h) {
  const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
  const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw >> 16, 1.0f, false);
  h[0] = lo[0]; h[1] = lo[1]; h[2] = hi[0]; h[3] = hi[1];
}

// Asynchronous copy of 16 bytes per lane into LDS through a buffer resource based at `base`
// (wave-uniform): lane i reads base + voff and writes lds + 16 i; vmcnt counts completion.
__device__ __forceinline__ void lds_copy16(const void* base, unsigned voff, void* lds) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_fp4_8(const float* q) {
  unsigned w = __float_as_uint(q[0]);  // every byte is written below; no register zeroing
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

// Half-precision offset of 16-byte chunk `ch` of row `row` in the K-hat tile (rows of D halves,
// chunk index XOR row mod D/8) and in the V-hat tile (rows of 128 halves, chunk index XOR a
// residue mixing the row's low and high bit pairs).
template <int D>
__device__ __forceinline__ int lds_k(int row, int ch) { return row * D + 8 * (ch ^ (row & (D / 8 - 1))); }
__device__ __forceinline__ int lds_v(int row, int ch) {
  return row * KV_TILE + 8 * (ch ^ (((row & 3) << 2) | ((row >> 2) & 3)));
}

// Online-softmax state of one 16-query group (per lane: one query, a quarter of its channels).
template <int D>
struct RowState {
  float m_u, R, l;  // running maximum and frame (log2 units), normaliser (sum of E in the frame)
  v4f O[D / 16];    // sum of P2-hat * V-hat in R's frame (P2 = 2688 E)
};

// One tile of the online softmax with the two-level P quantisation for one group. S holds the
// lane's 32 scores (masked ones -infinity); on return Pf holds P2-hat (fp16, code * s_P2) as the
// four B operands of the PV product, and O, l have been rescaled to this tile's reference.
template <int D>
__device__ __forceinline__ void softmax_tile(v4f* S, float k2, RowState<D>& st, v8h* Pf) {
  float bm[2];  // block maxima: a chain of three-input maxima over the block's 16 scores
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const v4f* B = S + 4 * h;
    const float a = max3f(B[0][0], B[0][1], B[0][2]), b = max3f(B[0][3], B[1][0], B[1][1]);
    const float c = max3f(B[1][2], B[1][3], B[2][0]), d = max3f(B[2][1], B[2][2], B[2][3]);
    const float e = max3f(B[3][0], B[3][1], B[3][2]);
    bm[h] = fmaxf(max3f(a, b, c), max3f(d, e, B[3][3]));
  }
  const float tS = xg_max(fmaxf(bm[0], bm[1]));
  const bool vis = tS > -INFINITY;
  // the exact tile maximum in log2 units, tau = tS*k2, is T + eT with T its FP32 rounding and eT
  // the rounding error (exact, |eT| <= ulp(T)/2). P and this tile's share of the normaliser take
  // tau as their frame, so that the maximal key has E = 1 exactly however large the scores (eT
  // matters only when ulp(T) does); between tiles the frames are rescaled by 2^(T_old - T), which
  // is as exact as the scores themselves are in FP32
  const float T = vis ? tS * k2 : 0.0f;
  const float eT = vis ? __builtin_fmaf(tS, k2, -T) : 0.0f;
  const float m_new = fmaxf(st.m_u, T);
  const bool accept = vis && (T >= m_new - 64.0f);
  const float bias = LOG2_2688 - T;  // log2(P2) = S*k2 + bias, up to the rounding of bias

  float sP[2], bq[2], wl[2];
  v2h sh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // block maximum of P2 = 2688 E with E = 2^(S*k2 - tau): the fma is exact for the block of
    // the tile maximum, whose argument is then exactly 0, so its P2 is 2688 as the two-level P
    // requires
    const float pmax = 2688.0f * __builtin_amdgcn_exp2f(__builtin_fmaf(bm[h], k2, -T) - eT);
    const unsigned sb = e4m3_encode(pmax * (1.0f / 6.0f));
    sP[h] = e4m3_decode(sb);
    bq[h] = sP[h] > 0.0f ? bias - __builtin_amdgcn_logf(sP[h]) : -INFINITY;  // log2(P2/s)
    // The quotients q = 2^(S*k2 + bq) carry the rounding of bq (up to an ulp of T, which moves
    // the code decisions only for huge scores): q = E * 2^(theta + eT) with E = 2^(S*k2 - tau)
    // and theta = T + bq, exact by Sterbenz. The block's share of the normaliser, sum E, is
    // therefore 2^-(theta + eT) * sum q, to a few ulp at any score magnitude.
    wl[h] = sP[h] > 0.0f ? __builtin_amdgcn_exp2f(-((T + bq[h]) + eT)) : 0.0f;
    // a rejected tile contributes nothing: its P blocks get scale 0 (codes are finite)
    const _Float16 s16 = accept ? (_Float16)sP[h] : (_Float16)0.0f;
    sh[h] = v2h{s16, s16};
  }
  float qsum[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int h = u >> 1;
    float q[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      q[jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * u + (jj >> 2)][jj & 3], k2, bq[h]));  // P2/s
      qsum[h] += q[jj];
    }
    Pf[u] = dequant8(pack_fp4_8(q), sh[h]);
  }
  const float lt = accept ? wl[0] * qsum[0] + wl[1] * qsum[1] : 0.0f;  // sum of E in T's frame
  const float factor = accept ? __builtin_amdgcn_exp2f(st.R - T) : 1.0f;
  st.R = accept ? T : st.R;
  st.m_u = m_new;
  st.l = st.l * factor + lt;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.O[dt] *= factor;
}

// KV16: kc is K-hat fp16 [BH][Np][D] and vc V-hat fp16 [BH][Np/128][D][128] (slot order), both
// zero past N; ks and vs are unused.
template <int D, bool CAUSAL, bool OUT_F32, bool KV16>
__global__ __launch_bounds__(256, 2) void attn_nvfp4_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
    int N, int64_t Np, int nqt, int nwork, int cgroup, float k2, void* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int KC = D / 8;        // 16-byte chunks per K-hat row (16 or 8)
  constexpr int CB = D / 4;        // code bytes each thread stages per tile, for K and for V
  constexpr int CW = CB / 4;       // ... in dwords (8 codes each; two dwords per 16-block)
  // LDS tiles with unpadded rows whose 16-byte chunks are XOR-swizzled per row (lds_k, lds_v).
  // The swizzles were chosen against gfx950's LDS banking as measured with the bank-conflict
  // counter: K's makes both the QK operand reads and the staging writes conflict-free, V's the
  // PV operand reads; V's staging lanes are grouped (below) so that its writes are too.
  __shared__ __attribute__((aligned(16))) _Float16 sK[KV_TILE * D];
  __shared__ __attribute__((aligned(16))) _Float16 sV[D * KV_TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int work = xcd_work((int)blockIdx.x, nwork);
  int64_t bh = work / nqt;
  int qt = work % nqt;
  if (CAUSAL) causal_work(work, nqt, nwork / nqt, cgroup, bh, qt);
  const int q0 = qt * NV_BQ;
  const int qi0 = q0 + 32 * w + c;  // group a holds query qi0 + 16a

  // Q-hat fragments (B operand of S^T = K Q^T): lane holds Q-hat[q][32kk + 8g .. +8).
  v8h qf[2][D / 32];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int qi = qi0 + 16 * a;
    const int64_t row = bh * N + qi;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      qf[a][kk] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      if (qi < N) {
        const unsigned wq = *reinterpret_cast<const unsigned*>(qc + row * (D / 2) + 16 * kk + 4 * g);
        const unsigned sb = qs[row * (D / 16) + 2 * kk + (g >> 1)];
        const _Float16 s16 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false)[0];
        qf[a][kk] = dequant8(wq, v2h{s16, s16});
      }
    }
  }

  RowState<D> st[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    st[a].m_u = -INFINITY; st[a].R = -INFINITY; st[a].l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st[a].O[dt] = v4f{0, 0, 0, 0};
  }

  // staging assignment: K row `kkey`, code bytes [kpart*CB, +CB); V channel `vd`, bytes
  // [vpart*CB, +CB) of the tile's 64. A write instruction is served eight consecutive lanes at a
  // time, which must hit distinct 16-byte slots modulo 128 bytes: with D = 128 eight consecutive
  // lanes take eight consecutive K rows; for V they take rows whose swizzle residues differ
  // (offsets 0, 1, 4, 5, 8, 9, 12, 13 of a 16-row group, or those plus 2).
  const int kkey = D == 128 ? 32 * w + (lane & 15) + 16 * (lane >> 5) : tid >> 1;
  const int kpart = D == 128 ? (lane >> 4) & 1 : tid & 1;
  const int vgrp = lane >> 3, vpos = lane & 7;
  const int vrow16 = (vpos & 1) + 4 * (vpos >> 1);
  const int vd = D == 128 ? 32 * w + 16 * (vgrp >> 2) + vrow16 + 2 * ((vgrp >> 1) & 1)
                          : 16 * w + vrow16 + 2 * (vgrp & 1);
  const int vpart = D == 128 ? vgrp & 1 : vgrp >> 1;
  // wave-uniform bases of this (batch, head); per-thread offsets stay 32-bit
  const uint8_t* kc_h = kc + bh * N * (D / 2);
  const uint8_t* ks_h = ks + bh * N * (D / 16);
  const uint8_t* vc_h = vc + bh * D * (Np / 2);
  const uint8_t* vs_h = vs + bh * D * (Np / 16);
  // V codes and scales are stored tile by tile, [Np/128][D][64] and [Np/128][D][8]
  const unsigned vc_off = (unsigned)(vd * 64 + vpart * CB);
  const unsigned vs_off = (unsigned)(vd * 8 + vpart * (CB / 8));
  unsigned kr[CW], vr[CW], ksr = 0, vsr = 0;

  auto prefetch = [&](int kt) {
    const int j = kt * KV_TILE + kkey;
    if (j < N) {
      const uint4* src = reinterpret_cast<const uint4*>(kc_h + (unsigned)(j * (D / 2) + kpart * CB));
#pragma unroll
      for (int u = 0; u < CW / 4; ++u) {
        const uint4 x = src[u];
        kr[4 * u] = x.x; kr[4 * u + 1] = x.y; kr[4 * u + 2] = x.z; kr[4 * u + 3] = x.w;
      }
      const uint8_t* sp = ks_h + (unsigned)(j * (D / 16) + kpart * (CB / 8));
      if (CB / 8 == 4) ksr = *reinterpret_cast<const unsigned*>(sp);
      else ksr = *reinterpret_cast<const unsigned short*>(sp);
    } else {
#pragma unroll
      for (int u = 0; u < CW; ++u) kr[u] = 0;
      ksr = 0;
    }
    const uint4* vsrc = reinterpret_cast<const uint4*>(vc_h + (vc_off + (unsigned)kt * (unsigned)(64 * D)));
#pragma unroll
    for (int u = 0; u < CW / 4; ++u) {
      const uint4 x = vsrc[u];
      vr[4 * u] = x.x; vr[4 * u + 1] = x.y; vr[4 * u + 2] = x.z; vr[4 * u + 3] = x.w;
    }
    const uint8_t* vsp = vs_h + (vs_off + (unsigned)kt * (unsigned)(8 * D));
    if (CB / 8 == 4) vsr = *reinterpret_cast<const unsigned*>(vsp);
    else vsr = *reinterpret_cast<const unsigned short*>(vsp);
  };

  // KV16 copies: job j of a wave fills bytes [1024 j, +1024) of the K-hat (V-hat) LDS tile, lane l
  // the 16 bytes at 1024 j + 16 l, i.e. one swizzled slot of one row, whose source is the row's
  // logical chunk (slot XOR the row's swizzle). The wave's share of a tile is JOBS copies; the row
  // part of a source offset is uniform, the rest depends on the job only through j mod 4.
  constexpr int JOBS = KV_TILE * D * 2 / 1024 / NV_WAVES;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, known to be uniform
  const uint8_t* kh_h = kc + bh * Np * (2 * D);
  const uint8_t* vh_h = vc + bh * Np * (2 * D);
  unsigned koff[4], voff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    koff[m] = D == 128 ? 256 * (lane >> 4) + 16 * ((lane & 15) ^ (4 * m + (lane >> 4)))
                       : 128 * (lane >> 3) + 16 * ((lane & 7) ^ ((lane >> 3) & 7));
    voff[m] = 256 * (lane >> 4) + 16 * ((lane & 15) ^ (((lane >> 4) << 2) | m));
  }
  auto copyK = [&](int kt) {
    const uint8_t* base = kh_h + (int64_t)kt * (KV_TILE * D * 2);
#pragma unroll
    for (int i = 0; i < JOBS; ++i) {
      const int j = wu * JOBS + i;
      lds_copy16(base + 1024 * j, koff[i & 3], reinterpret_cast<uint8_t*>(sK) + 1024 * j);
    }
  };
  auto copyV = [&](int kt) {
    const uint8_t* base = vh_h + (int64_t)kt * (KV_TILE * D * 2);
#pragma unroll
    for (int i = 0; i < JOBS; ++i) {
      const int j = wu * JOBS + i;
      lds_copy16(base + 1024 * j, voff[i & 3], reinterpret_cast<uint8_t*>(sV) + 1024 * j);
    }
  };

  const int ntiles = (int)(Np / KV_TILE);
  const int kt_end = CAUSAL ? min(ntiles, (q0 + NV_BQ - 1) / KV_TILE + 1) : ntiles;
  if constexpr (KV16) copyK(0);
  else prefetch(0);
  for (int kt = 0; kt < kt_end; ++kt) {
    if constexpr (KV16) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of K tile kt have landed
      __syncthreads();                // every wave's have, and every wave is done with V tile kt - 1
      copyV(kt);
    } else {
      __syncthreads();  // the previous tile's LDS reads are complete
      {
        _Float16 kh[4], vh[4];
        scales4(ksr, kh);
        scales4(vsr, vh);
#pragma unroll
        for (int u = 0; u < CW; ++u) {
          *reinterpret_cast<v8h*>(sK + lds_k<D>(kkey, CW * kpart + u)) = dequant8(kr[u], v2h{kh[u >> 1], kh[u >> 1]});
          *reinterpret_cast<v8h*>(sV + lds_v(vd, CW * vpart + u)) = dequant8(vr[u], v2h{vh[u >> 1], vh[u >> 1]});
        }
      }
      __syncthreads();
      if (kt + 1 < kt_end) prefetch(kt + 1);
    }
    // ---- S^T = K-hat Q-hat^T for both groups: subtile t covers keys 16t..16t+15. Operand
    // reads run two MFMA pairs ahead through a ring of three fragments.
    v4f S[2][8];
    {
      constexpr int NS = 8 * (D / 32);
      // row 16t + c, chunk 4kk + g; the swizzle depends on the row only through c
      auto kaddr = [&](int s) { return sK + 16 * (s / (D / 32)) * D + lds_k<D>(c, 4 * (s % (D / 32)) + g); };
      v8h f[3];
      f[0] = *reinterpret_cast<const v8h*>(kaddr(0));
      f[1] = *reinterpret_cast<const v8h*>(kaddr(1));
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        if (s2 + 2 < NS) f[(s2 + 2) % 3] = *reinterpret_cast<const v8h*>(kaddr(s2 + 2));
        const int t = s2 / (D / 32), kk = s2 % (D / 32);
        if (kk == 0) { S[0][t] = v4f{0, 0, 0, 0}; S[1][t] = v4f{0, 0, 0, 0}; }
        S[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[s2 % 3], qf[0][kk], S[0][t], 0, 0, 0);
        S[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[s2 % 3], qf[1][kk], S[1][t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- mask: keys past N, and keys after the query when causal
    const int kbase = kt * KV_TILE;
    if (kbase + KV_TILE > N || (CAUSAL && kbase + KV_TILE - 1 > q0)) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = kbase + 16 * t + 4 * g + i;
            if (j >= N || (CAUSAL && j > qi0 + 16 * a)) S[a][t][i] = -INFINITY;
          }
    }
    // ---- online softmax with the two-level quantisation of P, per group
    v8h Pf[2][4];
    softmax_tile<D>(S[0], k2, st[0], Pf[0]);
    softmax_tile<D>(S[1], k2, st[1], Pf[1]);
    if constexpr (KV16) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of V tile kt have landed
      __syncthreads();                // every wave's have, and every wave is done with K tile kt
      // unconditional, so that no branch splits the loop body (which costs registers): the last
      // tile copies itself again, into a buffer no wave reads any more
      copyK(min(kt + 1, kt_end - 1));
    }

    // ---- O^T += V-hat^T P-hat^T: MFMA step u covers slots 32g + 8u .. +8 of every lane group
    {
      constexpr int NS = D / 16 * 4;
      // row 16dt + c, chunk 4g + u; the swizzle depends on the row only through c
      auto vaddr = [&](int s) { return sV + 16 * (s >> 2) * KV_TILE + lds_v(c, 4 * g + (s & 3)); };
      v8h f[3];
      f[0] = *reinterpret_cast<const v8h*>(vaddr(0));
      f[1] = *reinterpret_cast<const v8h*>(vaddr(1));
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        if (s2 + 2 < NS) f[(s2 + 2) % 3] = *reinterpret_cast<const v8h*>(vaddr(s2 + 2));
        const int dt = s2 >> 2, u = s2 & 3;
        st[0].O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[s2 % 3], Pf[0][u], st[0].O[dt], 0, 0, 0);
        st[1].O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[s2 % 3], Pf[1][u], st[1].O[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if constexpr (KV16) __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the loop

  // ---- epilogue: O / (2688 l); lane (g, c) holds channels 16dt + 4g + i of its query in each
  // group. lse (when given): the row's log-sum-exp of the scaled scores, ln(2^R * l)
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const float L = xg_sum(st[a].l);
    const int qi = qi0 + 16 * a;
    if (qi < N) {
      const float inv = 1.0f / (2688.0f * L);
      const int64_t row = bh * N + qi;
      if (lse && g == 0) lse[row] = (st[a].R + __builtin_amdgcn_logf(L)) * 0.6931471805599453f;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const v4f o = st[a].O[dt] * inv;
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
}

template <int D, bool CAUSAL, bool F32, bool KV16>
static void launch_nv(const void* const* p, int BH, int N, float k2, void* out, float* lse, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const int nqt = (N + NV_BQ - 1) / NV_BQ;
  const int nwork = nqt * BH;
  // K and V bytes per head: codes + E4M3 scales, or fp16
  const int cgroup = causal_group(BH, KV16 ? Np * D * 4 : Np * D * 9 / 8);
  attn_nvfp4_kernel<D, CAUSAL, F32, KV16><<<dim3(nwork), dim3(64 * NV_WAVES), 0, st>>>(
      (const uint8_t*)p[0], (const uint8_t*)p[1], (const uint8_t*)p[2], (const uint8_t*)p[3],
      (const uint8_t*)p[4], (const uint8_t*)p[5], N, Np, nqt, nwork, cgroup, k2, out, lse);
}

// ptrs: Q codes, Q scales, K codes, K scales, V codes, V scales; with kv16, K-hat and V-hat fp16 in
// the places of the K and V codes (the scale pointers unused).
hipError_t launch_attn_nvfp4(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                             void* out, bool out_f32, float* lse, bool kv16, hipStream_t st) {
  const float k2 = sm_scale * 1.4426950408889634f;  // scores in log2 units
#define SAGE_NV_CASE(DD, CC, FF, KK) \
  if (D == DD && causal == CC && out_f32 == FF && kv16 == KK) launch_nv<DD, CC, FF, KK>(ptrs, BH, N, k2, out, lse, st);
#define SAGE_NV_CASES(KK)                                                                               \
  SAGE_NV_CASE(64, false, false, KK) SAGE_NV_CASE(64, false, true, KK) SAGE_NV_CASE(64, true, false, KK) \
  SAGE_NV_CASE(64, true, true, KK) SAGE_NV_CASE(128, false, false, KK) SAGE_NV_CASE(128, false, true, KK) \
  SAGE_NV_CASE(128, true, false, KK) SAGE_NV_CASE(128, true, true, KK)
  SAGE_NV_CASES(false)
  SAGE_NV_CASES(true)
#undef SAGE_NV_CASES
#undef SAGE_NV_CASE
  return hipGetLastError();
}

// K-hat fp16 [BH][Np][D] (rows past N zero) and V-hat fp16 [BH][Np/128][D][128] (the V codes'
// tile-major slot order; padding slots hold zero codes, so zero) from NVFP4 codes and scales.
// Block (x, bh): items x*256 + tid of head bh; item i < Np*D/8 writes eight K-hat values, the
// next Np*D/8 items eight V-hat values each. Every value is exact (code times E4M3 scale).
template <int D>
__global__ __launch_bounds__(256) void kv16_prep_kernel(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
                                                        const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
                                                        int N, int64_t Np, _Float16* __restrict__ kh,
                                                        _Float16* __restrict__ vh) {
  const int64_t bh = blockIdx.y, n8 = Np * (D / 8);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n8) return;
  if (i < n8) {
    const int64_t j = i / (D / 8);
    const int d = (int)(i % (D / 8)) * 8;
    v8h val = v8h{0, 0, 0, 0, 0, 0, 0, 0};
    if (j < N) {
      const int64_t r = bh * N + j;
      const unsigned w = *reinterpret_cast<const unsigned*>(kc + r * (D / 2) + d / 2);
      const _Float16 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ks[r * (D / 16) + d / 16], 1.0f, false)[0];
      val = dequant8(w, v2h{sc, sc});
    }
    *reinterpret_cast<v8h*>(kh + (bh * Np + j) * D + d) = val;
  } else {
    const int64_t e = bh * Np * D + 8 * (i - n8);  // element of [BH][Np/128][D][128]
    const unsigned w = *reinterpret_cast<const unsigned*>(vc + e / 2);
    const _Float16 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vs[e / 16], 1.0f, false)[0];
    *reinterpret_cast<v8h*>(vh + e) = dequant8(w, v2h{sc, sc});
  }
}

hipError_t launch_kv16_prep(const void* kc, const void* ks, const void* vc, const void* vs, int BH, int N, int D,
                            void* kv16, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  _Float16* kh = static_cast<_Float16*>(kv16);
  _Float16* vh = kh + (int64_t)BH * Np * D;
  const dim3 grid((unsigned)((2 * Np * (D / 8) + 255) / 256), (unsigned)BH);
  if (D == 64)
    kv16_prep_kernel<64><<<grid, dim3(256), 0, st>>>((const uint8_t*)kc, (const uint8_t*)ks, (const uint8_t*)vc,
                                                     (const uint8_t*)vs, N, Np, kh, vh);
  else
    kv16_prep_kernel<128><<<grid, dim3(256), 0, st>>>((const uint8_t*)kc, (const uint8_t*)ks, (const uint8_t*)vc,
                                                      (const uint8_t*)vs, N, Np, kh, vh);
  return hipGetLastError();
}

}  // namespace sage
