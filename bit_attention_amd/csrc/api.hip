// api.hip — the extern "C" boundary of libsage_fp4.so (declared in include/sage_fp4.h).
// Host-side argument validation happens before anything is enqueued; each entry point then
// launches exactly one kernel on the caller's stream and reports launch errors.
#include <cstdint>
#include <mutex>

#include "../../include/sage_fp4.h"
#include "device.h"

namespace sage {
hipError_t launch_quant_rows(bool mx, const void* x, int64_t rows, int D, void* codes, void* scales, hipStream_t st);
// vh: NULL, or (NVFP4) where V-hat goes; launch_quant_k_hat: NVFP4 K with K-hat at kh
hipError_t launch_quant_v(bool mx, const void* x, int BH, int N, int D, void* codes, void* scales, void* vh,
                          hipStream_t st);
hipError_t launch_quant_k_hat(const void* x, int BH, int N, int D, void* codes, void* scales, void* kh,
                              hipStream_t st);
hipError_t launch_quant_v8(const void* x, int BH, int N, int D, void* codes, void* scales, hipStream_t st);
// lse: NULL, or [B*H*N] fp32 that receives each row's log-sum-exp
// kv16: ptrs[2] and ptrs[4] are K-hat and V-hat in fp16 (sage_fp4_kv16_prep's layout)
hipError_t launch_attn_nvfp4(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                             void* out, bool out_f32, float* lse, bool kv16, hipStream_t st);
hipError_t launch_kv16_prep(const void* kc, const void* ks, const void* vc, const void* vs, int BH, int N, int D,
                            void* kv16, hipStream_t st);
hipError_t launch_attn_mxfp4(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                             void* out, bool out_f32, float* lse, hipStream_t st);
hipError_t launch_attn_mxfp4_direct_p(const void* const* ptrs, int BH, int N, int D, bool causal,
                                      float sm_scale, void* out, bool out_f32, float* lse, hipStream_t st);
hipError_t launch_attn_mx4_pv8(const void* const* ptrs, int BH, int N, int D, bool causal, float sm_scale,
                               void* out, bool out_f32, float* lse, hipStream_t st);
hipError_t launch_attn_bwd(int stages, bool mx, const void* qc, const void* qs, const void* kc, const void* ks,
                           const void* v, const void* o, const void* dout, const float* lse, int BH, int N, int D,
                           bool causal, float c, void* dq, void* dk, void* dv, bool out_f32, void* ws,
                           hipStream_t st);
size_t bwd_workspace_bytes(int64_t BH, int N, int D);
}  // namespace sage

namespace {

constexpr int kMaxN = 1 << 20;
// B*H*N*D < 2^36 keeps every launch grid below 2^32 work-items (the attention kernels run up to
// 4 work-items per query, the Q/K quantiser one per 16 elements); three fp16 tensors of that
// size would not fit in HBM anyway.
constexpr int64_t kMaxElems = int64_t(1) << 36;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_fmt(int fmt) { return fmt == SAGE_FMT_NVFP4 || fmt == SAGE_FMT_MXFP4 || fmt == SAGE_FMT_MX4_PV8; }

int check_shape(int B, int H, int N, int D) {
  if (D != 64 && D != 128) return SAGE_ERR_HEAD_DIM;
  if (B <= 0 || H <= 0 || N <= 0 || N > kMaxN) return SAGE_ERR_SHAPE;
  if ((int64_t)B * H > (int64_t)65535 || (int64_t)B * H * N * D >= kMaxElems) return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

int64_t padded(int N) { return ((int64_t)N + sage::KV_TILE - 1) / sage::KV_TILE * sage::KV_TILE; }

}  // namespace

extern "C" {

int sage_fp4_version(void) { return 500; }

int sage_fp4_kv_tile(void) { return sage::KV_TILE; }

int sage_fp4_slot_token(int slot) { return (slot < 0 || slot >= sage::KV_TILE) ? -1 : sage::slot_token(slot); }

size_t sage_fp4_codes_bytes(int role, int fmt, int B, int H, int N, int D) {
  if (check_shape(B, H, N, D) != SAGE_OK || !valid_fmt(fmt)) return 0;
  if (role == SAGE_ROLE_Q || role == SAGE_ROLE_K) return (size_t)B * H * N * (D / 2);
  if (role == SAGE_ROLE_V) return (size_t)B * H * D * (fmt == SAGE_FMT_MX4_PV8 ? padded(N) : padded(N) / 2);
  return 0;
}

size_t sage_fp4_scales_bytes(int role, int fmt, int B, int H, int N, int D) {
  if (check_shape(B, H, N, D) != SAGE_OK || !valid_fmt(fmt)) return 0;
  const int blk = fmt == SAGE_FMT_NVFP4 ? 16 : 32;
  if (role == SAGE_ROLE_Q || role == SAGE_ROLE_K) return (size_t)B * H * N * (D / blk);
  if (role == SAGE_ROLE_V) return (size_t)B * H * D * (padded(N) / blk);
  return 0;
}

int sage_fp4_quant(int role, int fmt, const void* x, int B, int H, int N, int D, void* codes, void* scales,
                   void* stream) {
  if (role != SAGE_ROLE_Q && role != SAGE_ROLE_K && role != SAGE_ROLE_V) return SAGE_ERR_ENUM;
  if (!valid_fmt(fmt)) return SAGE_ERR_ENUM;
  if (!x || !codes || !scales) return SAGE_ERR_NULL;
  const int sh = check_shape(B, H, N, D);
  if (sh != SAGE_OK) return sh;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return SAGE_ERR_ALIGN;
  const bool mx = fmt != SAGE_FMT_NVFP4;  // Q and K of the FP8-PV format are MXFP4
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (role == SAGE_ROLE_V && fmt == SAGE_FMT_MX4_PV8) e = sage::launch_quant_v8(x, B * H, N, D, codes, scales, st);
  else if (role == SAGE_ROLE_V) e = sage::launch_quant_v(mx, x, B * H, N, D, codes, scales, nullptr, st);
  else e = sage::launch_quant_rows(mx, x, (int64_t)B * H * N, D, codes, scales, st);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

// Validation shared by both attention entry points; SAGE_OK when the call may launch.
static int check_attn(const void* const* ptrs, int B, int H, int N, int D, const void* out, int out_dtype) {
  if (out_dtype != SAGE_OUT_F16 && out_dtype != SAGE_OUT_F32) return SAGE_ERR_ENUM;
  for (int i = 0; i < 6; ++i)
    if (!ptrs[i]) return SAGE_ERR_NULL;
  if (!out) return SAGE_ERR_NULL;
  const int sh = check_shape(B, H, N, D);
  if (sh != SAGE_OK) return sh;
  for (int i = 0; i < 6; ++i)
    if (!aligned16(ptrs[i])) return SAGE_ERR_ALIGN;
  if (!aligned16(out)) return SAGE_ERR_ALIGN;
  return SAGE_OK;
}

static float scale_or_default(float sm_scale, int D) {
  return sm_scale > 0.0f ? sm_scale : (float)(1.0 / __builtin_sqrt((double)D));
}

// One attention launch of any format; lse may be NULL (validated by the callers).
static int attn_any(int fmt, bool direct_p, const void* const* ptrs, int B, int H, int N, int D, int causal,
                    float sm_scale, void* out, int out_dtype, float* lse, void* stream) {
  const float c = scale_or_default(sm_scale, D);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool f32 = out_dtype == SAGE_OUT_F32, cz = causal != 0;
  const int BH = B * H;
  const hipError_t e = direct_p                  ? sage::launch_attn_mxfp4_direct_p(ptrs, BH, N, D, cz, c, out, f32, lse, st)
                       : fmt == SAGE_FMT_NVFP4   ? sage::launch_attn_nvfp4(ptrs, BH, N, D, cz, c, out, f32, lse, false, st)
                       : fmt == SAGE_FMT_MXFP4   ? sage::launch_attn_mxfp4(ptrs, BH, N, D, cz, c, out, f32, lse, st)
                                                 : sage::launch_attn_mx4_pv8(ptrs, BH, N, D, cz, c, out, f32, lse, st);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_fp4_attn_fwd(int fmt, const void* q_codes, const void* q_scales, const void* k_codes,
                      const void* k_scales, const void* v_codes, const void* v_scales, int B, int H, int N,
                      int D, int causal, float sm_scale, void* out, int out_dtype, void* stream) {
  if (!valid_fmt(fmt)) return SAGE_ERR_ENUM;
  const void* ptrs[6] = {q_codes, q_scales, k_codes, k_scales, v_codes, v_scales};
  const int chk = check_attn(ptrs, B, H, N, D, out, out_dtype);
  if (chk != SAGE_OK) return chk;
  return attn_any(fmt, false, ptrs, B, H, N, D, causal, sm_scale, out, out_dtype, nullptr, stream);
}

int sage_fp4_attn_fwd_direct_p(const void* q_codes, const void* q_scales, const void* k_codes,
                               const void* k_scales, const void* v_codes, const void* v_scales, int B, int H,
                               int N, int D, int causal, float sm_scale, void* out, int out_dtype,
                               void* stream) {
  const void* ptrs[6] = {q_codes, q_scales, k_codes, k_scales, v_codes, v_scales};
  const int chk = check_attn(ptrs, B, H, N, D, out, out_dtype);
  if (chk != SAGE_OK) return chk;
  return attn_any(SAGE_FMT_MXFP4, true, ptrs, B, H, N, D, causal, sm_scale, out, out_dtype, nullptr, stream);
}

int sage_fp4_attn_fwd_lse(int fmt, int direct_p, const void* q_codes, const void* q_scales, const void* k_codes,
                          const void* k_scales, const void* v_codes, const void* v_scales, int B, int H, int N,
                          int D, int causal, float sm_scale, void* out, int out_dtype, float* lse, void* stream) {
  if (!valid_fmt(fmt) || (direct_p != 0 && fmt != SAGE_FMT_MXFP4)) return SAGE_ERR_ENUM;
  const void* ptrs[6] = {q_codes, q_scales, k_codes, k_scales, v_codes, v_scales};
  const int chk = check_attn(ptrs, B, H, N, D, out, out_dtype);
  if (chk != SAGE_OK) return chk;
  if (!lse) return SAGE_ERR_NULL;
  if (!aligned16(lse)) return SAGE_ERR_ALIGN;
  return attn_any(fmt, direct_p != 0, ptrs, B, H, N, D, causal, sm_scale, out, out_dtype, lse, stream);
}

size_t sage_fp4_kv16_bytes(int B, int H, int N, int D) {
  if (check_shape(B, H, N, D) != SAGE_OK) return 0;
  return (size_t)4 * B * H * padded(N) * D;
}

int sage_fp4_kv16_prep(const void* k_codes, const void* k_scales, const void* v_codes, const void* v_scales, int B,
                       int H, int N, int D, void* kv16, size_t kv16_bytes, void* stream) {
  const void* ptrs[5] = {k_codes, k_scales, v_codes, v_scales, kv16};
  for (int i = 0; i < 5; ++i)
    if (!ptrs[i]) return SAGE_ERR_NULL;
  const int sh = check_shape(B, H, N, D);
  if (sh != SAGE_OK) return sh;
  for (int i = 0; i < 5; ++i)
    if (!aligned16(ptrs[i])) return SAGE_ERR_ALIGN;
  if (kv16_bytes < sage_fp4_kv16_bytes(B, H, N, D)) return SAGE_ERR_WORKSPACE;
  const hipError_t e = sage::launch_kv16_prep(k_codes, k_scales, v_codes, v_scales, B * H, N, D, kv16,
                                              reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_fp4_quant_kv16(int role, const void* x, int B, int H, int N, int D, void* codes, void* scales, void* kv16,
                        size_t kv16_bytes, void* stream) {
  if (role != SAGE_ROLE_K && role != SAGE_ROLE_V) return SAGE_ERR_ENUM;
  if (!x || !codes || !scales || !kv16) return SAGE_ERR_NULL;
  const int sh = check_shape(B, H, N, D);
  if (sh != SAGE_OK) return sh;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(kv16)) return SAGE_ERR_ALIGN;
  if (kv16_bytes < sage_fp4_kv16_bytes(B, H, N, D)) return SAGE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* kh = static_cast<uint8_t*>(kv16);
  const hipError_t e =
      role == SAGE_ROLE_K
          ? sage::launch_quant_k_hat(x, B * H, N, D, codes, scales, kh, st)
          : sage::launch_quant_v(false, x, B * H, N, D, codes, scales, kh + (size_t)2 * B * H * padded(N) * D, st);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_fp4_attn_fwd_kv16(const void* q_codes, const void* q_scales, const void* kv16, size_t kv16_bytes, int B,
                           int H, int N, int D, int causal, float sm_scale, void* out, int out_dtype, float* lse,
                           void* stream) {
  if (out_dtype != SAGE_OUT_F16 && out_dtype != SAGE_OUT_F32) return SAGE_ERR_ENUM;
  if (!q_codes || !q_scales || !kv16 || !out) return SAGE_ERR_NULL;
  const int sh = check_shape(B, H, N, D);
  if (sh != SAGE_OK) return sh;
  if (!aligned16(q_codes) || !aligned16(q_scales) || !aligned16(kv16) || !aligned16(out) || !aligned16(lse))
    return SAGE_ERR_ALIGN;
  if (kv16_bytes < sage_fp4_kv16_bytes(B, H, N, D)) return SAGE_ERR_WORKSPACE;
  const uint8_t* kh = static_cast<const uint8_t*>(kv16);
  const uint8_t* vh = kh + (size_t)2 * B * H * padded(N) * D;
  const void* ptrs[6] = {q_codes, q_scales, kh, nullptr, vh, nullptr};
  const hipError_t e =
      sage::launch_attn_nvfp4(ptrs, B * H, N, D, causal != 0, scale_or_default(sm_scale, D), out,
                              out_dtype == SAGE_OUT_F32, lse, true, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

size_t sage_fp4_attn_bwd_workspace_bytes(int B, int H, int N, int D) {
  if (check_shape(B, H, N, D) != SAGE_OK) return 0;
  return sage::bwd_workspace_bytes((int64_t)B * H, N, D);
}

// Validation of the backward's arguments other than the workspace; SAGE_OK when they are valid.
static int check_bwd(int fmt, const void* const* in, int B, int H, int N, int D, int out_dtype) {
  if (!valid_fmt(fmt) || (out_dtype != SAGE_OUT_F16 && out_dtype != SAGE_OUT_F32)) return SAGE_ERR_ENUM;
  for (int i = 0; i < 11; ++i)
    if (!in[i]) return SAGE_ERR_NULL;
  const int sh = check_shape(B, H, N, D);
  if (sh != SAGE_OK) return sh;
  for (int i = 0; i < 11; ++i)
    if (!aligned16(in[i])) return SAGE_ERR_ALIGN;
  return SAGE_OK;
}

static int launch_bwd(int stages, int fmt, const void* const* in, int B, int H, int N, int D, int causal,
                      float sm_scale, int out_dtype, void* workspace, void* stream) {
  const hipError_t e = sage::launch_attn_bwd(stages, fmt != SAGE_FMT_NVFP4, in[0], in[1], in[2], in[3], in[4], in[5],
                                             in[6], static_cast<const float*>(in[7]), B * H, N, D, causal != 0,
                                             scale_or_default(sm_scale, D), const_cast<void*>(in[8]),
                                             const_cast<void*>(in[9]), const_cast<void*>(in[10]),
                                             out_dtype == SAGE_OUT_F32, workspace, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

// The backward, all stages (mask 7) or one (1 prep, 2 dK/dV, 4 dQ).
static int attn_bwd_stages(int stages, int fmt, const void* q_codes, const void* q_scales, const void* k_codes,
                           const void* k_scales, const void* v, const void* o, const void* dout, const float* lse,
                           int B, int H, int N, int D, int causal, float sm_scale, void* dq, void* dk, void* dv,
                           int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const void* in[11] = {q_codes, q_scales, k_codes, k_scales, v, o, dout, lse, dq, dk, dv};
  const int chk = check_bwd(fmt, in, B, H, N, D, out_dtype);
  if (chk != SAGE_OK) return chk;
  if (!workspace) return SAGE_ERR_NULL;
  if (!aligned16(workspace)) return SAGE_ERR_ALIGN;
  if (workspace_bytes < sage::bwd_workspace_bytes((int64_t)B * H, N, D)) return SAGE_ERR_WORKSPACE;
  return launch_bwd(stages, fmt, in, B, H, N, D, causal, sm_scale, out_dtype, workspace, stream);
}

int sage_fp4_attn_bwd(int fmt, const void* q_codes, const void* q_scales, const void* k_codes, const void* k_scales,
                      const void* v, const void* o, const void* dout, const float* lse, int B, int H, int N, int D,
                      int causal, float sm_scale, void* dq, void* dk, void* dv, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return attn_bwd_stages(7, fmt, q_codes, q_scales, k_codes, k_scales, v, o, dout, lse, B, H, N, D, causal, sm_scale,
                         dq, dk, dv, out_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the backward without allocation: its workspace is a device-resident array of this file ----

// One copy per GPU, held until the process ends. Host code never uses the name as an address:
// the kernels get the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[SAGE_BWD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device, set on first use

// The address of `scratch` on the device that runs `stream` (the current device for the null
// stream), looked up once per device with that device current.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0, cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" int sage_fp4_attn_bwd_noalloc(int fmt, const void* q_codes, const void* q_scales, const void* k_codes,
                                         const void* k_scales, const void* v, const void* o, const void* dout,
                                         const float* lse, int B, int H, int N, int D, int causal, float sm_scale,
                                         void* dq, void* dk, void* dv, int out_dtype, void* stream) {
  const void* in[11] = {q_codes, q_scales, k_codes, k_scales, v, o, dout, lse, dq, dk, dv};
  const int chk = check_bwd(fmt, in, B, H, N, D, out_dtype);
  if (chk != SAGE_OK) return chk;
  if (sage::bwd_workspace_bytes((int64_t)B * H, N, D) > SAGE_BWD_NOALLOC_SCRATCH_BYTES) return SAGE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(reinterpret_cast<hipStream_t>(stream), &ws) != hipSuccess) return SAGE_ERR_HIP;
  return launch_bwd(7, fmt, in, B, H, N, D, causal, sm_scale, out_dtype, ws, stream);
}

extern "C" {

int sage_fp4_attn_bwd_stage(int stage, int fmt, const void* q_codes, const void* q_scales, const void* k_codes,
                            const void* k_scales, const void* v, const void* o, const void* dout, const float* lse,
                            int B, int H, int N, int D, int causal, float sm_scale, void* dq, void* dk, void* dv,
                            int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage != SAGE_BWD_PREP && stage != SAGE_BWD_DKDV && stage != SAGE_BWD_DQ) return SAGE_ERR_ENUM;
  return attn_bwd_stages(1 << stage, fmt, q_codes, q_scales, k_codes, k_scales, v, o, dout, lse, B, H, N, D, causal,
                         sm_scale, dq, dk, dv, out_dtype, workspace, workspace_bytes, stream);
}

const char* sage_fp4_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_NULL: return "a required pointer is NULL";
    case SAGE_ERR_SHAPE: return "B, H or N out of range";
    case SAGE_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case SAGE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SAGE_ERR_ENUM: return "bad format, role or output type";
    case SAGE_ERR_HIP: return "HIP runtime error at launch";
    case SAGE_ERR_WORKSPACE: return "workspace smaller than the call needs";
    default: return "unknown status";
  }
}

}  // extern "C"
