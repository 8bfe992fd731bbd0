"""ctypes binding of libsage_fp4.so (include/sage_fp4.h). Argument marshalling only: every step
of the computation runs in the library's HIP kernels. PyTorch supplies device memory and streams.

The functions named like the C entry points take raw pointers/ints; the convenience wrappers
(`quant`, `attn_fwd`, `attn_bwd_into`) take torch tensors and pass the current stream."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsage_fp4.so")

NVFP4, MXFP4, MX4_PV8 = 0, 1, 2
ROLE_Q, ROLE_K, ROLE_V = 0, 1, 2
OUT_F16, OUT_F32 = 0, 1
BWD_PREP, BWD_DKDV, BWD_DQ = 0, 1, 2
STATUS = {0: "SAGE_OK", -1: "SAGE_ERR_NULL", -2: "SAGE_ERR_SHAPE", -3: "SAGE_ERR_HEAD_DIM",
          -4: "SAGE_ERR_ALIGN", -5: "SAGE_ERR_ENUM", -6: "SAGE_ERR_HIP", -7: "SAGE_ERR_WORKSPACE"}
EXPORTS = ["sage_fp4_version", "sage_fp4_kv_tile", "sage_fp4_slot_token", "sage_fp4_codes_bytes",
           "sage_fp4_scales_bytes", "sage_fp4_quant", "sage_fp4_attn_fwd", "sage_fp4_attn_fwd_direct_p",
           "sage_fp4_attn_fwd_lse", "sage_fp4_attn_bwd_workspace_bytes", "sage_fp4_attn_bwd",
           "sage_fp4_attn_bwd_stage", "sage_fp4_status_string"]

_lib = None


class SageError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")
        self.status = status


def lib():
    """Load the library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python -m bit_attention_amd.build")
        L = C.CDLL(LIB_PATH)
        I, P, F, S = C.c_int, C.c_void_p, C.c_float, C.c_size_t
        L.sage_fp4_version.argtypes = []; L.sage_fp4_version.restype = I
        L.sage_fp4_kv_tile.argtypes = []; L.sage_fp4_kv_tile.restype = I
        L.sage_fp4_slot_token.argtypes = [I]; L.sage_fp4_slot_token.restype = I
        L.sage_fp4_codes_bytes.argtypes = [I, I, I, I, I, I]; L.sage_fp4_codes_bytes.restype = S
        L.sage_fp4_scales_bytes.argtypes = [I, I, I, I, I, I]; L.sage_fp4_scales_bytes.restype = S
        L.sage_fp4_quant.argtypes = [I, I, P, I, I, I, I, P, P, P]; L.sage_fp4_quant.restype = I
        L.sage_fp4_attn_fwd.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, F, P, I, P]
        L.sage_fp4_attn_fwd.restype = I
        L.sage_fp4_attn_fwd_direct_p.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, P, I, P]
        L.sage_fp4_attn_fwd_direct_p.restype = I
        L.sage_fp4_attn_fwd_lse.argtypes = [I, I, P, P, P, P, P, P, I, I, I, I, I, F, P, I, P, P]
        L.sage_fp4_attn_fwd_lse.restype = I
        L.sage_fp4_attn_bwd_workspace_bytes.argtypes = [I, I, I, I]
        L.sage_fp4_attn_bwd_workspace_bytes.restype = S
        L.sage_fp4_attn_bwd.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, P, P, I, P, S, P]
        L.sage_fp4_attn_bwd.restype = I
        L.sage_fp4_attn_bwd_stage.argtypes = [I] + L.sage_fp4_attn_bwd.argtypes
        L.sage_fp4_attn_bwd_stage.restype = I
        L.sage_fp4_status_string.argtypes = [I]; L.sage_fp4_status_string.restype = C.c_char_p
        _lib = L
    return _lib


# ---- the C entry points, same names, raw arguments ----
def sage_fp4_version() -> int:
    return lib().sage_fp4_version()


def sage_fp4_kv_tile() -> int:
    return lib().sage_fp4_kv_tile()


def sage_fp4_slot_token(slot: int) -> int:
    return lib().sage_fp4_slot_token(slot)


def sage_fp4_codes_bytes(role, fmt, B, H, N, D) -> int:
    return lib().sage_fp4_codes_bytes(role, fmt, B, H, N, D)


def sage_fp4_scales_bytes(role, fmt, B, H, N, D) -> int:
    return lib().sage_fp4_scales_bytes(role, fmt, B, H, N, D)


def sage_fp4_quant(role, fmt, x_ptr, B, H, N, D, codes_ptr, scales_ptr, stream_ptr) -> int:
    return lib().sage_fp4_quant(role, fmt, x_ptr, B, H, N, D, codes_ptr, scales_ptr, stream_ptr)


def sage_fp4_attn_fwd(fmt, qc, qs, kc, ks, vc, vs, B, H, N, D, causal, sm_scale, out_ptr, out_dtype,
                      stream_ptr) -> int:
    return lib().sage_fp4_attn_fwd(fmt, qc, qs, kc, ks, vc, vs, B, H, N, D, int(causal), float(sm_scale),
                                   out_ptr, out_dtype, stream_ptr)


def sage_fp4_attn_fwd_direct_p(qc, qs, kc, ks, vc, vs, B, H, N, D, causal, sm_scale, out_ptr, out_dtype,
                               stream_ptr) -> int:
    return lib().sage_fp4_attn_fwd_direct_p(qc, qs, kc, ks, vc, vs, B, H, N, D, int(causal), float(sm_scale),
                                            out_ptr, out_dtype, stream_ptr)


def sage_fp4_attn_fwd_lse(fmt, direct_p, qc, qs, kc, ks, vc, vs, B, H, N, D, causal, sm_scale, out_ptr,
                          out_dtype, lse_ptr, stream_ptr) -> int:
    return lib().sage_fp4_attn_fwd_lse(fmt, int(direct_p), qc, qs, kc, ks, vc, vs, B, H, N, D, int(causal),
                                       float(sm_scale), out_ptr, out_dtype, lse_ptr, stream_ptr)


def sage_fp4_attn_bwd_workspace_bytes(B, H, N, D) -> int:
    return lib().sage_fp4_attn_bwd_workspace_bytes(B, H, N, D)


def sage_fp4_attn_bwd(fmt, qc, qs, kc, ks, v_ptr, o_ptr, do_ptr, lse_ptr, B, H, N, D, causal, sm_scale,
                      dq_ptr, dk_ptr, dv_ptr, out_dtype, ws_ptr, ws_bytes, stream_ptr) -> int:
    return lib().sage_fp4_attn_bwd(fmt, qc, qs, kc, ks, v_ptr, o_ptr, do_ptr, lse_ptr, B, H, N, D, int(causal),
                                   float(sm_scale), dq_ptr, dk_ptr, dv_ptr, out_dtype, ws_ptr, ws_bytes,
                                   stream_ptr)


def sage_fp4_attn_bwd_stage(stage, fmt, qc, qs, kc, ks, v_ptr, o_ptr, do_ptr, lse_ptr, B, H, N, D, causal,
                            sm_scale, dq_ptr, dk_ptr, dv_ptr, out_dtype, ws_ptr, ws_bytes, stream_ptr) -> int:
    return lib().sage_fp4_attn_bwd_stage(stage, fmt, qc, qs, kc, ks, v_ptr, o_ptr, do_ptr, lse_ptr, B, H, N, D,
                                         int(causal), float(sm_scale), dq_ptr, dk_ptr, dv_ptr, out_dtype, ws_ptr,
                                         ws_bytes, stream_ptr)


def status_string(status: int) -> str:
    return lib().sage_fp4_status_string(status).decode()


# ---- torch conveniences ----
def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(t, dtype, what):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (ROCm) tensor")
    if t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous {dtype} tensor")


def alloc_quant(role, fmt, B, H, N, D, device="cuda"):
    import torch
    nc = sage_fp4_codes_bytes(role, fmt, B, H, N, D)
    ns = sage_fp4_scales_bytes(role, fmt, B, H, N, D)
    if nc == 0 or ns == 0:
        raise SageError(-2, "sage_fp4_codes_bytes")
    return (torch.empty(nc, dtype=torch.uint8, device=device),
            torch.empty(ns, dtype=torch.uint8, device=device))


def quant_into(x, role, fmt, codes, scales, stream=None):
    import torch
    _check(x, torch.float16, "x")
    B, H, N, D = x.shape
    rc = sage_fp4_quant(role, fmt, C.c_void_p(x.data_ptr()), B, H, N, D, C.c_void_p(codes.data_ptr()),
                        C.c_void_p(scales.data_ptr()), _stream_ptr(stream))
    if rc != 0:
        raise SageError(rc, "sage_fp4_quant")
    return codes, scales


def quant(x, role, fmt, stream=None):
    """x: fp16 CUDA tensor [B,H,N,D] -> (codes, scales) uint8 CUDA tensors (flat)."""
    B, H, N, D = x.shape
    codes, scales = alloc_quant(role, fmt, B, H, N, D, device=x.device)
    return quant_into(x, role, fmt, codes, scales, stream)


def _out_code(out):
    import torch
    if out.dtype == torch.float32:
        return OUT_F32
    if out.dtype == torch.float16:
        return OUT_F16
    raise TypeError("out must be float16 or float32")


def attn_fwd_into(fmt, q, k, v, shape, out, causal=False, sm_scale=0.0, stream=None, direct_p=False, lse=None):
    """direct_p=True calls sage_fp4_attn_fwd_direct_p (MXFP4 operands only); a float32 tensor
    `lse` of B*H*N elements calls sage_fp4_attn_fwd_lse, which also writes each row's
    log-sum-exp."""
    import torch
    B, H, N, D = shape
    od = _out_code(out)
    ptrs = [C.c_void_p(t.data_ptr()) for pair in (q, k, v) for t in pair]
    if lse is not None:
        _check(lse, torch.float32, "lse")
        if lse.numel() != B * H * N:
            raise ValueError("lse must hold B*H*N elements")
        rc = sage_fp4_attn_fwd_lse(fmt, direct_p, *ptrs, B, H, N, D, causal, sm_scale, C.c_void_p(out.data_ptr()),
                                   od, C.c_void_p(lse.data_ptr()), _stream_ptr(stream))
        what = "sage_fp4_attn_fwd_lse"
    elif direct_p:
        if fmt != MXFP4:
            raise ValueError("Direct-P takes MXFP4 operands")
        rc = sage_fp4_attn_fwd_direct_p(*ptrs, B, H, N, D, causal, sm_scale, C.c_void_p(out.data_ptr()), od,
                                        _stream_ptr(stream))
        what = "sage_fp4_attn_fwd_direct_p"
    else:
        rc = sage_fp4_attn_fwd(fmt, *ptrs, B, H, N, D, causal, sm_scale, C.c_void_p(out.data_ptr()), od,
                               _stream_ptr(stream))
        what = "sage_fp4_attn_fwd"
    if rc != 0:
        raise SageError(rc, what)
    return out


def attn_fwd(fmt, q, k, v, shape, causal=False, sm_scale=0.0, out_dtype=None, stream=None, direct_p=False):
    """q, k, v: (codes, scales) pairs from quant(); returns out [B,H,N,D]."""
    import torch
    dt = torch.float32 if out_dtype is None else out_dtype
    out = torch.empty(shape, dtype=dt, device=q[0].device)
    return attn_fwd_into(fmt, q, k, v, shape, out, causal, sm_scale, stream, direct_p)


def alloc_bwd_workspace(B, H, N, D, device="cuda"):
    import torch
    n = sage_fp4_attn_bwd_workspace_bytes(B, H, N, D)
    if n == 0:
        raise SageError(-2, "sage_fp4_attn_bwd_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_bwd_into(fmt, q, k, v, o, do, lse, dq, dk, dv, workspace, causal=False, sm_scale=0.0, stream=None,
                  stage=None):
    """q, k: (codes, scales) pairs of the forward's Q and K; v, o, do: fp16 [B,H,N,D]; lse: fp32
    with B*H*N elements; dq, dk, dv: outputs of one dtype (fp16 or fp32); workspace: uint8 of at
    least sage_fp4_attn_bwd_workspace_bytes bytes. Calls sage_fp4_attn_bwd, or with `stage`
    (BWD_PREP, BWD_DKDV, BWD_DQ) sage_fp4_attn_bwd_stage."""
    import torch
    for t, n in ((v, "v"), (o, "o"), (do, "do")):
        _check(t, torch.float16, n)
    _check(lse, torch.float32, "lse")
    B, H, N, D = v.shape
    if o.shape != v.shape or do.shape != v.shape or lse.numel() != B * H * N:
        raise ValueError("o and do must match v's shape and lse must hold B*H*N elements")
    od = _out_code(dq)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, dq.dtype, n)
        if t.shape != v.shape:
            raise ValueError(f"{n} must have v's shape")
    args = [C.c_void_p(t.data_ptr()) for pair in (q, k) for t in pair]
    args += [C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()), C.c_void_p(do.data_ptr()),
             C.c_void_p(lse.data_ptr()), B, H, N, D, causal, sm_scale, C.c_void_p(dq.data_ptr()),
             C.c_void_p(dk.data_ptr()), C.c_void_p(dv.data_ptr()), od, C.c_void_p(workspace.data_ptr()),
             workspace.numel(), _stream_ptr(stream)]
    if stage is None:
        rc, what = sage_fp4_attn_bwd(fmt, *args), "sage_fp4_attn_bwd"
    else:
        rc, what = sage_fp4_attn_bwd_stage(stage, fmt, *args), "sage_fp4_attn_bwd_stage"
    if rc != 0:
        raise SageError(rc, what)
    return dq, dk, dv
