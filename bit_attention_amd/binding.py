"""ctypes binding of libsage_fp4.so (include/sage_fp4.h). Argument marshalling only: every step
of the computation runs in the library's HIP kernels. PyTorch supplies device memory and streams.

The functions named like the C entry points take raw pointers/ints; the convenience wrappers
(`quant`, `attn_fwd`, `kv16_prep`, `quant_kv16`, `quant_kv16_into`, `attn_fwd_kv16_into`,
`attn_bwd_into`) take torch tensors and
pass the current stream."""
from __future__ import annotations

import ctypes as C
import functools
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsage_fp4.so")

NVFP4, MXFP4, MX4_PV8 = 0, 1, 2
ROLE_Q, ROLE_K, ROLE_V = 0, 1, 2
OUT_F16, OUT_F32 = 0, 1
BWD_PREP, BWD_DKDV, BWD_DQ = 0, 1, 2
STATUS = {0: "SAGE_OK", -1: "SAGE_ERR_NULL", -2: "SAGE_ERR_SHAPE", -3: "SAGE_ERR_HEAD_DIM",
          -4: "SAGE_ERR_ALIGN", -5: "SAGE_ERR_ENUM", -6: "SAGE_ERR_HIP", -7: "SAGE_ERR_WORKSPACE"}
ERR_SHAPE = -2  # SAGE_ERR_SHAPE: raised here when a size query returns 0 for the shape
EXPORTS = ["sage_fp4_version", "sage_fp4_kv_tile", "sage_fp4_slot_token", "sage_fp4_codes_bytes",
           "sage_fp4_scales_bytes", "sage_fp4_quant", "sage_fp4_attn_fwd", "sage_fp4_attn_fwd_direct_p",
           "sage_fp4_attn_fwd_lse", "sage_fp4_kv16_bytes", "sage_fp4_kv16_prep", "sage_fp4_quant_kv16",
           "sage_fp4_attn_fwd_kv16",
           "sage_fp4_attn_bwd_workspace_bytes", "sage_fp4_attn_bwd",
           "sage_fp4_attn_bwd_stage", "sage_fp4_attn_bwd_noalloc", "sage_fp4_status_string"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # SAGE_BWD_NOALLOC_SCRATCH_BYTES

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
        L.sage_fp4_kv16_bytes.argtypes = [I, I, I, I]; L.sage_fp4_kv16_bytes.restype = S
        L.sage_fp4_kv16_prep.argtypes = [P, P, P, P, I, I, I, I, P, S, P]; L.sage_fp4_kv16_prep.restype = I
        L.sage_fp4_quant_kv16.argtypes = [I, P, I, I, I, I, P, P, P, S, P]; L.sage_fp4_quant_kv16.restype = I
        L.sage_fp4_attn_fwd_kv16.argtypes = [P, P, P, S, I, I, I, I, I, F, P, I, P, P]
        L.sage_fp4_attn_fwd_kv16.restype = I
        L.sage_fp4_attn_bwd_workspace_bytes.argtypes = [I, I, I, I]
        L.sage_fp4_attn_bwd_workspace_bytes.restype = S
        L.sage_fp4_attn_bwd.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, P, P, I, P, S, P]
        L.sage_fp4_attn_bwd.restype = I
        L.sage_fp4_attn_bwd_stage.argtypes = [I] + L.sage_fp4_attn_bwd.argtypes
        L.sage_fp4_attn_bwd_stage.restype = I
        L.sage_fp4_attn_bwd_noalloc.argtypes = L.sage_fp4_attn_bwd.argtypes[:19] + [P]
        L.sage_fp4_attn_bwd_noalloc.restype = I
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


@functools.lru_cache(maxsize=256)
def _sizes(role, fmt, B, H, N, D):
    """(codes, scales) bytes for one operand, cached: the wrappers check sizes on every call."""
    return sage_fp4_codes_bytes(role, fmt, B, H, N, D), sage_fp4_scales_bytes(role, fmt, B, H, N, D)


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


def sage_fp4_kv16_bytes(B, H, N, D) -> int:
    return lib().sage_fp4_kv16_bytes(B, H, N, D)


def sage_fp4_kv16_prep(kc, ks, vc, vs, B, H, N, D, kv16_ptr, kv16_bytes, stream_ptr) -> int:
    return lib().sage_fp4_kv16_prep(kc, ks, vc, vs, B, H, N, D, kv16_ptr, kv16_bytes, stream_ptr)


def sage_fp4_quant_kv16(role, x_ptr, B, H, N, D, codes_ptr, scales_ptr, kv16_ptr, kv16_bytes, stream_ptr) -> int:
    return lib().sage_fp4_quant_kv16(role, x_ptr, B, H, N, D, codes_ptr, scales_ptr, kv16_ptr, kv16_bytes,
                                     stream_ptr)


def sage_fp4_attn_fwd_kv16(qc, qs, kv16_ptr, kv16_bytes, B, H, N, D, causal, sm_scale, out_ptr, out_dtype,
                           lse_ptr, stream_ptr) -> int:
    return lib().sage_fp4_attn_fwd_kv16(qc, qs, kv16_ptr, kv16_bytes, B, H, N, D, int(causal), float(sm_scale),
                                        out_ptr, out_dtype, lse_ptr, stream_ptr)


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


def sage_fp4_attn_bwd_noalloc(fmt, qc, qs, kc, ks, v_ptr, o_ptr, do_ptr, lse_ptr, B, H, N, D, causal, sm_scale,
                              dq_ptr, dk_ptr, dv_ptr, out_dtype, stream_ptr) -> int:
    return lib().sage_fp4_attn_bwd_noalloc(fmt, qc, qs, kc, ks, v_ptr, o_ptr, do_ptr, lse_ptr, B, H, N, D,
                                           int(causal), float(sm_scale), dq_ptr, dk_ptr, dv_ptr, out_dtype,
                                           stream_ptr)


def status_string(status: int) -> str:
    return lib().sage_fp4_status_string(status).decode()


# ---- torch conveniences ----
def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _on_gpu(t) -> bool:
    return t.is_cuda


def _check(t, dtype, what, device=None, min_numel=None, numel=None):
    """t must be a contiguous CUDA (ROCm) tensor of `dtype`, on `device` when given, with at least
    `min_numel` (or exactly `numel`) elements: the C ABI cannot see buffer sizes, so an undersized
    buffer would otherwise be read or written out of bounds by the kernels."""
    import torch
    if not isinstance(t, torch.Tensor) or not _on_gpu(t):
        raise TypeError(f"{what} must be a CUDA (ROCm) tensor")
    if t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous {dtype} tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, the other operands on {device}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{what} holds {t.numel()} elements, the call needs {min_numel}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what} holds {t.numel()} elements, the call needs exactly {numel}")


def _check_codes(pair, role, fmt, shape, device, what):
    """A (codes, scales) pair of `role` in format `fmt` for shape (B, H, N, D)."""
    import torch
    if not isinstance(pair, (tuple, list)) or len(pair) != 2:
        raise TypeError(f"{what} must be a (codes, scales) pair")
    B, H, N, D = shape
    nc, ns = _sizes(role, fmt, B, H, N, D)
    if nc == 0 or ns == 0:
        raise SageError(ERR_SHAPE, f"{what}: shape {shape}")
    _check(pair[0], torch.uint8, f"{what} codes", device, min_numel=nc)
    _check(pair[1], torch.uint8, f"{what} scales", device, min_numel=ns)


def alloc_quant(role, fmt, B, H, N, D, device="cuda"):
    import torch
    nc = sage_fp4_codes_bytes(role, fmt, B, H, N, D)
    ns = sage_fp4_scales_bytes(role, fmt, B, H, N, D)
    if nc == 0 or ns == 0:
        raise SageError(ERR_SHAPE, "sage_fp4_codes_bytes")
    return (torch.empty(nc, dtype=torch.uint8, device=device),
            torch.empty(ns, dtype=torch.uint8, device=device))


def quant_into(x, role, fmt, codes, scales, stream=None):
    import torch
    _check(x, torch.float16, "x")
    if x.dim() != 4:
        raise ValueError("x must be [B,H,N,D]")
    B, H, N, D = x.shape
    _check_codes((codes, scales), role, fmt, (B, H, N, D), x.device, "output")
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
    dev = q[0].device if isinstance(q, (tuple, list)) and len(q) == 2 else None
    for pair, role, name in ((q, ROLE_Q, "q"), (k, ROLE_K, "k"), (v, ROLE_V, "v")):
        _check_codes(pair, role, fmt, shape, dev, name)
    _check(out, out.dtype, "out", dev, numel=B * H * N * D)
    ptrs = [C.c_void_p(t.data_ptr()) for pair in (q, k, v) for t in pair]
    if lse is not None:
        _check(lse, torch.float32, "lse", dev, numel=B * H * N)
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


def kv16_prep(k, v, shape, kv16=None, stream=None):
    """k, v: NVFP4 (codes, scales) pairs from quant(); returns the uint8 buffer (allocated unless
    `kv16` is given) holding K-hat and V-hat in fp16, as sage_fp4_kv16_prep writes it."""
    import torch
    B, H, N, D = shape
    dev = k[0].device if isinstance(k, (tuple, list)) and len(k) == 2 else None
    for pair, role, name in ((k, ROLE_K, "k"), (v, ROLE_V, "v")):
        _check_codes(pair, role, NVFP4, shape, dev, name)
    need = sage_fp4_kv16_bytes(B, H, N, D)
    if kv16 is None:
        kv16 = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(kv16, torch.uint8, "kv16", dev, min_numel=need)
    ptrs = [C.c_void_p(t.data_ptr()) for pair in (k, v) for t in pair]
    rc = sage_fp4_kv16_prep(*ptrs, B, H, N, D, C.c_void_p(kv16.data_ptr()), kv16.numel(), _stream_ptr(stream))
    if rc != 0:
        raise SageError(rc, "sage_fp4_kv16_prep")
    return kv16


def quant_kv16_into(x, role, codes, scales, kv16, stream=None):
    """x: fp16 CUDA tensor [B,H,N,D] (K for role ROLE_K, V for ROLE_V) -> its NVFP4 codes and
    scales (as quant_into writes them) and its half of `kv16` (as kv16_prep writes it), by one
    sage_fp4_quant_kv16 call."""
    import torch
    _check(x, torch.float16, "x")
    if x.dim() != 4:
        raise ValueError("x must be [B,H,N,D]")
    if role not in (ROLE_K, ROLE_V):
        raise ValueError("role must be ROLE_K or ROLE_V")
    B, H, N, D = x.shape
    _check_codes((codes, scales), role, NVFP4, (B, H, N, D), x.device, "output")
    _check(kv16, torch.uint8, "kv16", x.device, min_numel=sage_fp4_kv16_bytes(B, H, N, D))
    rc = sage_fp4_quant_kv16(role, C.c_void_p(x.data_ptr()), B, H, N, D, C.c_void_p(codes.data_ptr()),
                             C.c_void_p(scales.data_ptr()), C.c_void_p(kv16.data_ptr()), kv16.numel(),
                             _stream_ptr(stream))
    if rc != 0:
        raise SageError(rc, "sage_fp4_quant_kv16")
    return codes, scales


def quant_kv16(k, v, kv16=None, stream=None):
    """k, v: fp16 CUDA tensors [B,H,N,D] -> (K pair, V pair, kv16): the NVFP4 (codes, scales) pairs
    quant() would return and the buffer kv16_prep() would fill from them (allocated unless `kv16`
    is given)."""
    import torch
    _check(k, torch.float16, "k")
    if k.dim() != 4:
        raise ValueError("k must be [B,H,N,D]")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k {tuple(k.shape)}")
    B, H, N, D = k.shape
    need = sage_fp4_kv16_bytes(B, H, N, D)
    if need == 0:
        raise SageError(ERR_SHAPE, f"sage_fp4_kv16_bytes: shape {tuple(k.shape)}")
    if kv16 is None:
        kv16 = torch.empty(need, dtype=torch.uint8, device=k.device)
    K = quant_kv16_into(k, ROLE_K, *alloc_quant(ROLE_K, NVFP4, B, H, N, D, device=k.device), kv16, stream)
    V = quant_kv16_into(v, ROLE_V, *alloc_quant(ROLE_V, NVFP4, B, H, N, D, device=k.device), kv16, stream)
    return K, V, kv16


def attn_fwd_kv16_into(q, kv16, shape, out, causal=False, sm_scale=0.0, stream=None, lse=None):
    """q: NVFP4 (codes, scales) pair; kv16: the buffer from kv16_prep or quant_kv16; out [B,H,N,D]
    fp16 or fp32; lse: None or float32 with B*H*N elements. Calls sage_fp4_attn_fwd_kv16."""
    import torch
    B, H, N, D = shape
    od = _out_code(out)
    dev = q[0].device if isinstance(q, (tuple, list)) and len(q) == 2 else None
    _check_codes(q, ROLE_Q, NVFP4, shape, dev, "q")
    _check(kv16, torch.uint8, "kv16", dev, min_numel=sage_fp4_kv16_bytes(B, H, N, D))
    _check(out, out.dtype, "out", dev, numel=B * H * N * D)
    lse_ptr = None
    if lse is not None:
        _check(lse, torch.float32, "lse", dev, numel=B * H * N)
        lse_ptr = C.c_void_p(lse.data_ptr())
    rc = sage_fp4_attn_fwd_kv16(C.c_void_p(q[0].data_ptr()), C.c_void_p(q[1].data_ptr()),
                                C.c_void_p(kv16.data_ptr()), kv16.numel(), B, H, N, D, causal, sm_scale,
                                C.c_void_p(out.data_ptr()), od, lse_ptr, _stream_ptr(stream))
    if rc != 0:
        raise SageError(rc, "sage_fp4_attn_fwd_kv16")
    return out


def alloc_bwd_workspace(B, H, N, D, device="cuda"):
    import torch
    n = sage_fp4_attn_bwd_workspace_bytes(B, H, N, D)
    if n == 0:
        raise SageError(ERR_SHAPE, "sage_fp4_attn_bwd_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _bwd_args(fmt, q, k, v, o, do, lse, dq, dk, dv, causal, sm_scale):
    """Checked raw arguments of the backward entry points, up to out_dtype."""
    import torch
    _check(v, torch.float16, "v")
    if v.dim() != 4:
        raise ValueError("v must be [B,H,N,D]")
    B, H, N, D = v.shape
    dev = v.device
    for t, n in ((o, "o"), (do, "do")):
        _check(t, torch.float16, n, dev, numel=v.numel())
        if t.shape != v.shape:
            raise ValueError(f"{n} must have v's shape")
    _check(lse, torch.float32, "lse", dev, numel=B * H * N)
    for pair, role, name in ((q, ROLE_Q, "q"), (k, ROLE_K, "k")):
        _check_codes(pair, role, fmt, (B, H, N, D), dev, name)
    od = _out_code(dq)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, dq.dtype, n, dev, numel=v.numel())
        if t.shape != v.shape:
            raise ValueError(f"{n} must have v's shape")
    args = [C.c_void_p(t.data_ptr()) for pair in (q, k) for t in pair]
    args += [C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()), C.c_void_p(do.data_ptr()),
             C.c_void_p(lse.data_ptr()), B, H, N, D, causal, sm_scale, C.c_void_p(dq.data_ptr()),
             C.c_void_p(dk.data_ptr()), C.c_void_p(dv.data_ptr()), od]
    return args, dev, (B, H, N, D)


def attn_bwd_into(fmt, q, k, v, o, do, lse, dq, dk, dv, workspace, causal=False, sm_scale=0.0, stream=None,
                  stage=None):
    """q, k: (codes, scales) pairs of the forward's Q and K; v, o, do: fp16 [B,H,N,D]; lse: fp32
    with B*H*N elements; dq, dk, dv: outputs of one dtype (fp16 or fp32); workspace: uint8 of at
    least sage_fp4_attn_bwd_workspace_bytes bytes. Calls sage_fp4_attn_bwd, or with `stage`
    (BWD_PREP, BWD_DKDV, BWD_DQ) sage_fp4_attn_bwd_stage."""
    import torch
    args, dev, (B, H, N, D) = _bwd_args(fmt, q, k, v, o, do, lse, dq, dk, dv, causal, sm_scale)
    _check(workspace, torch.uint8, "workspace", dev, min_numel=sage_fp4_attn_bwd_workspace_bytes(B, H, N, D))
    args += [C.c_void_p(workspace.data_ptr()), workspace.numel(), _stream_ptr(stream)]
    if stage is None:
        rc, what = sage_fp4_attn_bwd(fmt, *args), "sage_fp4_attn_bwd"
    else:
        rc, what = sage_fp4_attn_bwd_stage(stage, fmt, *args), "sage_fp4_attn_bwd_stage"
    if rc != 0:
        raise SageError(rc, what)
    return dq, dk, dv


def attn_bwd_noalloc_into(fmt, q, k, v, o, do, lse, dq, dk, dv, causal=False, sm_scale=0.0, stream=None):
    """As attn_bwd_into without a workspace: calls sage_fp4_attn_bwd_noalloc, whose workspace is
    the library's device-resident array (SAGE_ERR_WORKSPACE for shapes that do not fit it)."""
    args, _, _ = _bwd_args(fmt, q, k, v, o, do, lse, dq, dk, dv, causal, sm_scale)
    rc = sage_fp4_attn_bwd_noalloc(fmt, *args, _stream_ptr(stream))
    if rc != 0:
        raise SageError(rc, "sage_fp4_attn_bwd_noalloc")
    return dq, dk, dv
