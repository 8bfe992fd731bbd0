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
// NVFP4 operands are dequantised exactly to fp16 (code * 2^e by the hardware conversion, times
// the 1+m/8 mantissa by one fp16 multiply) and both products run on v_mfma_f32_16x16x32_f16.
//   - workgroup = 8 waves = 128 queries of one (batch, head); key tiles of 128.
//   - K and V of a tile are staged in LDS once per workgroup, dequantised to fp16.
//   - each wave computes S^T = K Q^T for its 16 queries: after 8 subtiles a lane holds the 32
//     scores of one query at keys 16t + 4g + i, exactly the slot order the quantisation kernel
//     stores V in, so P's 1x16 blocks are lane-local (two per lane per tile), their maxima come
//     out of the row-max pass, and the quantised P is already the B operand of O^T = V^T P^T.
//   - the row max needs two cross-lane swaps (permlane16/32); everything else is lane-local.
//   - accumulator reference: O and l are kept relative to the current tile's maximum, so the
//     MFMA accumulates P2-hat * V-hat directly; one multiply rescales them per tile. A tile whose
//     maximum lies more than 2^64 below the running maximum is dropped for that row (relative
//     weight below 2^-64).
#include "device.h"

namespace sage {

constexpr int NV_WAVES = 8;
constexpr int NV_BQ = 16 * NV_WAVES;
constexpr float LOG2_2688 = 11.392317422778762f;  // log2(448 * 6)

__device__ __forceinline__ v8h dequant8(unsigned w, float p2, v2h mu) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 0) * mu;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 1) * mu;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 2) * mu;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 3) * mu;
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E4M3 scale byte -> (2^floor(log2 s), 1+m/8 as an fp16 pair); s == 0 gives (1, 0).
__device__ __forceinline__ void split_scale(unsigned sb, float* p2, v2h* mu) {
  const float s = e4m3_decode(sb);
  *p2 = pow2_floor(s);
  const _Float16 m = (_Float16)(s / *p2);
  *mu = v2h{m, m};
}

__device__ __forceinline__ unsigned pack_fp4_8(const float* q) {
  unsigned w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(512) void attn_nvfp4_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
    int N, int64_t Np, int nqt, float k2, void* __restrict__ out) {
  constexpr int KP = D + 8;        // K-hat row pitch (halves)
  constexpr int VP = KV_TILE + 8;  // V-hat row pitch (halves)
  constexpr int CH = D / 8;        // code bytes per thread per tile, for K and for V
  __shared__ __attribute__((aligned(16))) _Float16 sK[KV_TILE * KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[D * VP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.x) : (int)blockIdx.x;  // heavy tiles first
  const int64_t bh = blockIdx.y;
  const int q0 = qt * NV_BQ;
  const int qi = q0 + 16 * w + c;  // this lane's query

  // Q-hat fragments (B operand of S^T = K Q^T): lane holds Q-hat[qi][32kk + 8g .. +8).
  v8h qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    qf[kk] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
    if (qi < N) {
      const int64_t row = bh * N + qi;
      const unsigned wq = *reinterpret_cast<const unsigned*>(qc + row * (D / 2) + 16 * kk + 4 * g);
      float p2; v2h mu;
      split_scale(qs[row * (D / 16) + 2 * kk + (g >> 1)], &p2, &mu);
      qf[kk] = dequant8(wq, p2, mu);
    }
  }

  float m_u = -INFINITY, R = -INFINITY, l2 = 0.0f;
  v4f O[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) O[dt] = v4f{0, 0, 0, 0};

  const int ntiles = (int)(Np / KV_TILE);
  const int kt_end = CAUSAL ? min(ntiles, (q0 + NV_BQ - 1) / KV_TILE + 1) : ntiles;
  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();  // the previous tile's LDS reads are complete
    {
      // K: thread -> (key, part): CH code bytes = 2*CH codes = CH/8 blocks of 16
      const int key = tid / 4, part = tid % 4;
      const int j = kt * KV_TILE + key;
      _Float16* dst = sK + key * KP + part * 2 * CH;
      if (j < N) {
        const int64_t row = bh * N + j;
        const unsigned* src = reinterpret_cast<const unsigned*>(kc + row * (D / 2) + part * CH);
#pragma unroll
        for (int u = 0; u < CH / 4; ++u) {
          float p2; v2h mu;
          split_scale(ks[row * (D / 16) + (part * 2 * CH + 8 * u) / 16], &p2, &mu);
          *reinterpret_cast<v8h*>(dst + 8 * u) = dequant8(src[u], p2, mu);
        }
      } else {
#pragma unroll
        for (int u = 0; u < CH / 4; ++u) *reinterpret_cast<v8h*>(dst + 8 * u) = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    {
      // V: codes [D][Np/2]; thread -> (channel, part): CH bytes = 2*CH slots
      constexpr int TPR = 64 / CH;  // threads per channel row
      const int d = tid / TPR, part = tid % TPR;
      const int64_t vrow = bh * D + d;
      const unsigned* src = reinterpret_cast<const unsigned*>(vc + vrow * (Np / 2) + (int64_t)kt * 64 + part * CH);
      _Float16* dst = sV + d * VP + part * 2 * CH;
#pragma unroll
      for (int u = 0; u < CH / 4; ++u) {
        float p2; v2h mu;
        split_scale(vs[vrow * (Np / 16) + (int64_t)kt * 8 + (part * 2 * CH + 8 * u) / 16], &p2, &mu);
        *reinterpret_cast<v8h*>(dst + 8 * u) = dequant8(src[u], p2, mu);
      }
    }
    __syncthreads();

    // ---- S^T = K-hat Q-hat^T for 16 queries: subtile t covers keys 16t..16t+15
    v4f S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      S[t] = v4f{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const v8h a = *reinterpret_cast<const v8h*>(sK + (16 * t + c) * KP + 32 * kk + 8 * g);
        S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[kk], S[t], 0, 0, 0);
      }
    }
    // ---- mask: keys past N, and keys after the query when causal
    const int kbase = kt * KV_TILE;
    if (kbase + KV_TILE > N || (CAUSAL && kbase + KV_TILE - 1 > q0)) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kbase + 16 * t + 4 * g + i;
          if (j >= N || (CAUSAL && j > qi)) S[t][i] = -INFINITY;
        }
    }
    // ---- online softmax with the two-level quantisation of P
    float bm[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 4 * h; t < 4 * h + 4; ++t)
        mx = fmaxf(fmaxf(mx, fmaxf(S[t][0], S[t][1])), fmaxf(S[t][2], S[t][3]));
      bm[h] = mx;
    }
    const float tS = xg_max(fmaxf(bm[0], bm[1]));
    const bool vis = tS > -INFINITY;
    const float t_u = tS * k2;  // tile maximum in log2 units
    const float m_new = fmaxf(m_u, t_u);
    const bool accept = vis && (t_u >= m_new - 64.0f);
    const float bias = vis ? LOG2_2688 - t_u : -INFINITY;  // log2(P2) = S*k2 + bias

    float sP[2], bq[2], p2s[2];
    v2h mus[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float pmax = __builtin_amdgcn_exp2f(__builtin_fmaf(bm[h], k2, bias));  // block max of P2
      const unsigned sb = e4m3_encode(pmax * (1.0f / 6.0f));
      sP[h] = e4m3_decode(sb);
      bq[h] = sP[h] > 0.0f ? bias - __builtin_amdgcn_logf(sP[h]) : -INFINITY;  // log2(P2/s)
      p2s[h] = pow2_floor(sP[h]);
      const _Float16 m = (_Float16)(sP[h] / p2s[h]);
      mus[h] = v2h{m, m};
    }
    float qsum[2] = {0.0f, 0.0f};
    v8h Pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int h = u >> 1;
      float q[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        q[jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * u + (jj >> 2)][jj & 3], k2, bq[h]));  // P2/s
        qsum[h] += q[jj];
      }
      Pf[u] = dequant8(pack_fp4_8(q), p2s[h], mus[h]);
    }
    float l2t = sP[0] * qsum[0] + sP[1] * qsum[1];
    if (!accept) {
      l2t = 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u) Pf[u] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const float factor = accept ? __builtin_amdgcn_exp2f(R - t_u) : 1.0f;
    R = accept ? t_u : R;
    m_u = m_new;
    l2 = l2 * factor + l2t;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[dt] *= factor;

    // ---- O^T += V-hat^T P-hat^T: MFMA step u covers slots 32g + 8u .. +8 of every lane group
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v8h a = *reinterpret_cast<const v8h*>(sV + (16 * dt + c) * VP + 32 * g + 8 * u);
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, Pf[u], O[dt], 0, 0, 0);
      }
  }

  // ---- epilogue: O / l; lane (g, c) holds channels 16dt + 4g + i of query qi
  const float L = xg_sum(l2);
  if (qi < N) {
    const float inv = 1.0f / L;
    const int64_t row = bh * N + qi;
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

template <int D, bool CAUSAL, bool F32>
static void launch_nv(const void* const* p, int BH, int N, float k2, void* out, hipStream_t st) {
  const int64_t Np = ((int64_t)N + KV_TILE - 1) / KV_TILE * KV_TILE;
  const int nqt = (N + NV_BQ - 1) / NV_BQ;
  attn_nvfp4_kernel<D, CAUSAL, F32><<<dim3(nqt, BH), dim3(512), 0, st>>>(
      (const uint8_t*)p[0], (const uint8_t*)p[1], (const uint8_t*)p[2], (const uint8_t*)p[3],
      (const uint8_t*)p[4], (const uint8_t*)p[5], N, Np, nqt, k2, out);
}

hipError_t launch_attn_nvfp4(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                             void* out, bool out_f32, hipStream_t st) {
  const float k2 = sm_scale * 1.4426950408889634f;  // scores in log2 units
#define SAGE_NV_CASE(DD, CC, FF) \
  if (D == DD && causal == CC && out_f32 == FF) launch_nv<DD, CC, FF>(ptrs, BH, N, k2, out, st);
  SAGE_NV_CASE(64, false, false) SAGE_NV_CASE(64, false, true) SAGE_NV_CASE(64, true, false)
  SAGE_NV_CASE(64, true, true) SAGE_NV_CASE(128, false, false) SAGE_NV_CASE(128, false, true)
  SAGE_NV_CASE(128, true, false) SAGE_NV_CASE(128, true, true)
#undef SAGE_NV_CASE
  return hipGetLastError();
}

}  // namespace sage
