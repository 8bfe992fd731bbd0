"""CPU oracle for microscaling-FP4 attention (forward) — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The GPU library never uses it; the two share no code. The arithmetic lives
in ``sage_oracle.c`` (plain C, FP32 in the method's order); this module only marshals numpy
arrays through ctypes.

Source: SageAttention3 (arXiv 2505.11594), DeepTech article sections on the two FP4 obstacles
(1x16 microscaling, two-level P quantisation into [0, 448*6]) and on FP4 data types (NVFP4 =
E2M1/1x16/E4M3, MXFP4 = E2M1/1x32/E8M0) and the fused online softmax.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsage_oracle.so")
SRC = os.path.join(HERE, "sage_oracle.c")

NVFP4, MXFP4, MX4_PV8 = 0, 1, 2  # MX4_PV8: MXFP4 Q/K, MXFP8 (E4M3, 1x32, E8M0) P and V
ROLE_Q, ROLE_K, ROLE_V = 0, 1, 2
KV_TILE = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", SRC,
               "-o", LIB_PATH, "-lm"]
        subprocess.run(cmd, check=True)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        P, I, I64, F, D = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_double
        L.orc_f16_to_f32.argtypes = [C.c_uint16]; L.orc_f16_to_f32.restype = F
        L.orc_e2m1_decode.argtypes = [C.c_uint]; L.orc_e2m1_decode.restype = F
        L.orc_e4m3_decode.argtypes = [C.c_uint]; L.orc_e4m3_decode.restype = F
        L.orc_e8m0_decode.argtypes = [C.c_uint]; L.orc_e8m0_decode.restype = F
        L.orc_e4m3_encode.argtypes = [F]; L.orc_e4m3_encode.restype = C.c_uint
        L.orc_e2m1_quant.argtypes = [F, F]; L.orc_e2m1_quant.restype = C.c_uint
        L.orc_mx_scale.argtypes = [F]; L.orc_mx_scale.restype = C.c_uint
        L.orc_mx8_scale.argtypes = [F]; L.orc_mx8_scale.restype = C.c_uint
        L.orc_e4m3_quant.argtypes = [F, F]; L.orc_e4m3_quant.restype = C.c_uint
        L.orc_slot_token.argtypes = [I]; L.orc_slot_token.restype = I
        L.orc_e4m3_encode_many.argtypes = [P, I64, P]; L.orc_e4m3_encode_many.restype = None
        L.orc_e2m1_quant_many.argtypes = [P, P, I64, P]; L.orc_e2m1_quant_many.restype = None
        L.orc_quant_block_nv.argtypes = [P, I, P, P]; L.orc_quant_block_nv.restype = None
        L.orc_quant_block_mx.argtypes = [P, I, P, P]; L.orc_quant_block_mx.restype = None
        L.orc_quant_block_mx8.argtypes = [P, I, P, P]; L.orc_quant_block_mx8.restype = None
        L.orc_quant.argtypes = [I, I, P, I, I, I, I, P, P]; L.orc_quant.restype = I
        L.orc_p_tile.argtypes = [I, P, P, P, P, P, P]; L.orc_p_tile.restype = I
        L.orc_attn_fwd.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, F, P, I64, P, P, D, I]
        L.orc_attn_fwd.restype = I
        L.orc_attn_fwd_direct_p.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, P, I64, P, P, D, I]
        L.orc_attn_fwd_direct_p.restype = I
        L.orc_attn_fwd_lse.argtypes = [I, I, P, P, P, P, P, P, I, I, I, I, I, F, P, I64, P, P, P, P, D, I]
        L.orc_attn_fwd_lse.restype = I
        L.orc_attn_ref_f64.argtypes = [P, P, P, I, I, I, I, I, D, P, I64, P, I]
        L.orc_attn_ref_f64.restype = I
        L.orc_max_threads.argtypes = []; L.orc_max_threads.restype = I
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def blk(fmt: int) -> int:
    return 16 if fmt == NVFP4 else 32


def padded_n(N: int) -> int:
    return (N + KV_TILE - 1) // KV_TILE * KV_TILE


def quant(role: int, fmt: int, x: np.ndarray):
    """x: float16 array [B,H,N,D] -> (codes uint8, scales uint8) in the documented layouts."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    B, H, N, D = x.shape
    b = blk(fmt)
    if role == ROLE_V:
        Np = padded_n(N)
        codes = np.zeros((B, H, Np // KV_TILE, D, KV_TILE if fmt == MX4_PV8 else KV_TILE // 2), np.uint8)
        scales = np.zeros((B, H, Np // KV_TILE, D, KV_TILE // b), np.uint8)
    else:
        codes = np.zeros((B, H, N, D // 2), np.uint8)
        scales = np.zeros((B, H, N, D // b), np.uint8)
    rc = lib().orc_quant(role, fmt, _p(x.view(np.uint16)), B, H, N, D, _p(codes), _p(scales))
    if rc != 0:
        raise ValueError(f"orc_quant failed ({rc})")
    return codes, scales


def attn_fwd(fmt, q, k, v, shape, causal=False, sm_scale=0.0, rows=None, want_slack=False,
             delta=2.0 ** -14, nthreads=0, direct_p=False, want_lse=False):
    """q, k, v: (codes, scales) tuples from quant(); shape = (B,H,N,D). direct_p selects the
    Direct-P normaliser (MXFP4 operands only).

    Returns out float32 ([B,H,N,D], or [len(rows), D]); if want_slack, then per-row slack; if
    want_lse, then the per-row log-sum-exp (float64, [B*H*N] or [len(rows)]) and, with
    want_slack too, its per-row slack."""
    if direct_p and fmt != MXFP4:
        raise ValueError("Direct-P takes MXFP4 operands")
    B, H, N, D = shape
    arrs = [np.ascontiguousarray(a) for t in (q, k, v) for a in t]
    if rows is None:
        out = np.empty((B, H, N, D), np.float32)
        rp, nr = None, 0
        nslack = B * H * N
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((len(rows), D), np.float32)
        rp, nr = _p(rows), len(rows)
        nslack = len(rows)
    slack = np.zeros(nslack, np.float64) if want_slack else None
    if want_lse:
        lse = np.zeros(nslack, np.float64)
        lse_slack = np.zeros(nslack, np.float64) if want_slack else None
        rc = lib().orc_attn_fwd_lse(fmt, int(direct_p), *[_p(a) for a in arrs], B, H, N, D, int(causal),
                                    float(sm_scale), rp, nr, _p(out), _p(lse), _p(slack) if want_slack else None,
                                    _p(lse_slack) if want_slack else None, float(delta), int(nthreads))
        if rc != 0:
            raise ValueError(f"orc_attn_fwd_lse failed ({rc})")
        return (out, slack, lse, lse_slack) if want_slack else (out, lse)
    tail = (B, H, N, D, int(causal), float(sm_scale), rp, nr, _p(out), _p(slack) if want_slack else None,
            float(delta), int(nthreads))
    if direct_p:
        rc = lib().orc_attn_fwd_direct_p(*[_p(a) for a in arrs], *tail)
    else:
        rc = lib().orc_attn_fwd(fmt, *[_p(a) for a in arrs], *tail)
    if rc != 0:
        raise ValueError(f"orc_attn_fwd failed ({rc})")
    return (out, slack) if want_slack else out


def attn_ref_f64(q, k, v, causal=False, sm_scale=0.0, rows=None, nthreads=0):
    """Unquantised softmax(c Q K^T) V in double from fp16 inputs [B,H,N,D]."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float16) for a in (q, k, v))
    B, H, N, D = q.shape
    if rows is None:
        out = np.empty((B, H, N, D), np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((len(rows), D), np.float64)
        rp, nr = _p(rows), len(rows)
    rc = lib().orc_attn_ref_f64(_p(q.view(np.uint16)), _p(k.view(np.uint16)), _p(v.view(np.uint16)),
                                B, H, N, D, int(causal), float(sm_scale), rp, nr, _p(out), int(nthreads))
    if rc != 0:
        raise ValueError(f"orc_attn_ref_f64 failed ({rc})")
    return out


def p_tile(fmt, x: np.ndarray, vis: np.ndarray):
    """One (row, tile) of P. Returns (E, codes, scales, t) or None if nothing is visible."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    vis = np.ascontiguousarray(vis, dtype=np.uint8)
    E = np.zeros(KV_TILE, np.float32)
    codes = np.zeros(KV_TILE, np.uint8)
    scales = np.zeros(KV_TILE // blk(fmt), np.uint8)
    t = np.zeros(1, np.float32)
    ok = lib().orc_p_tile(fmt, _p(x), _p(vis), _p(E), _p(codes), _p(scales), _p(t))
    return (E, codes, scales, float(t[0])) if ok else None


def e4m3_encode_many(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e4m3_encode_many(_p(y), y.size, _p(out))
    return out


def e2m1_quant_many(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.ascontiguousarray(np.broadcast_to(s, x.shape), dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e2m1_quant_many(_p(x), _p(s), x.size, _p(out))
    return out


def quant_block(fmt, x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(len(x), np.uint8)
    s = np.zeros(1, np.uint8)
    f = {NVFP4: lib().orc_quant_block_nv, MXFP4: lib().orc_quant_block_mx, MX4_PV8: lib().orc_quant_block_mx8}[fmt]
    f(_p(x), len(x), _p(codes), _p(s))
    return codes, int(s[0])


# ---- dequantisation helpers (decode through the oracle's own codec tables) ----
def e2m1_table() -> np.ndarray:
    return np.array([lib().orc_e2m1_decode(c) for c in range(16)], np.float32)


def scale_table(fmt) -> np.ndarray:
    f = lib().orc_e4m3_decode if fmt == NVFP4 else lib().orc_e8m0_decode
    return np.array([f(b) for b in range(256)], np.float32)


def unpack(codes: np.ndarray) -> np.ndarray:
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def e4m3_table() -> np.ndarray:
    return np.array([lib().orc_e4m3_decode(b) for b in range(256)], np.float32)


def dequant(fmt, codes, scales) -> np.ndarray:
    """Values code*scale (float64) along the last axis. With MX4_PV8 the codes are the FP8 bytes
    of V (or P); its Q and K codes are MXFP4 and dequantise with fmt = MXFP4. V's codes and
    scales go through v_by_channel() first."""
    if np.ndim(codes) != np.ndim(scales) or np.ndim(codes) > 4:
        raise ValueError("codes and scales must be [..., rows, cols] alike (V: use v_by_channel first)")
    if fmt == MX4_PV8:
        c = e4m3_table()[codes].astype(np.float64)
    else:
        c = e2m1_table()[unpack(codes)].astype(np.float64)
    s = scale_table(fmt)[scales].astype(np.float64)
    return c * np.repeat(s, blk(fmt), axis=-1)


def _tiles_to_rows(a: np.ndarray) -> np.ndarray:
    B, H, T, D, w = a.shape
    return np.ascontiguousarray(np.transpose(a, (0, 1, 3, 2, 4))).reshape(B, H, D, T * w)


def v_by_channel(codes: np.ndarray, scales: np.ndarray):
    """V's codes and scales from their stored tile-by-tile layouts ([B,H,Np/128,D,64 or 128] and
    [B,H,Np/128,D,128/blk]) to one row per channel ([B,H,D,Np/2 or Np] and [B,H,D,Np/blk]),
    slot positions in order along the row: the form dequant() takes."""
    return _tiles_to_rows(codes), _tiles_to_rows(scales)


def slot_tokens() -> np.ndarray:
    return np.array([lib().orc_slot_token(s) for s in range(KV_TILE)], np.int64)


def max_threads() -> int:
    return lib().orc_max_threads()
