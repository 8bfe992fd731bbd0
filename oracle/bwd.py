"""CPU oracle for the 8-bit attention backward — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module. The GPU library never uses it and shares no code with it.

What it computes. SageAttention3 (arXiv 2505.11594; DeepTech article, sections on the third
difficulty and on INT8 attention for training) runs six of the seven matmuls of attention
training in INT8 and keeps the backward one most sensitive to precision in 16 bits; the
sensitive quantity is the gradient of the attention map. The rit.work page on FP4
FlashAttention-4 (section "What was done") has the forward hand the backward its quantized Q
and K, their scales and the normaliser. The pages name no granularities. The reading (R16):

  S    = Q^ K^T            exactly, from the forward's FP4 Q^ and K^ (dequantised values)
  P    = exp(c S - lse)    lse from the forward; 0 where the key is not visible
  dP   = dO V^T            16-bit operands (fp16 dO and V), the matmul kept out of INT8
  D_i  = sum_d dO_id O_id
  dS   = P * (dP - D)
  dV   = P^T dO            INT8
  dK   = c dS^T Q^         INT8
  dQ   = c dS K^           INT8

Each INT8 operand has one fp32 scale per row (the index that is not contracted) and per block
of 64 consecutive contraction indices: P^T and dS^T per (key, 64-query block); dS for dQ per
(query, 64-key block); dO, Q^ and K^ per (channel, 64-token block). An INT8 matmul is then a
sum over contraction blocks of an exact integer product times the two scales.

INT8 encoding of the 64 values x of one (row, block), a = max|x|, all in fp32 (the kernel's
precision, since the decisions are integers): scale = fl32(a / 127), r = fl32(127 / a),
code = rne(fl32(x * r)) clamped to [-127, 127]; a = 0 gives scale 0 and codes 0. Tokens past N
are zero.

Everything else is float64: S, P, dP, D and dS from the exact operands, so a correct kernel
differs only by its float32 rounding, except where a rounding decision (a P or dS code) lies
within that rounding of its boundary. With ``want_bounds`` the oracle returns, per output
element, ``slack``: the sum of the largest effect of every such ambiguous decision (the
kernel may round it either way), of the scale's own float32 error, and of whole blocks whose
maximum is itself at rounding-noise level (``_slack_mag``), and ``mag``: the sum of the
magnitudes of the terms of the element, on which a float32 tolerance is scaled.
"""
from __future__ import annotations

import numpy as np

from . import MX4_PV8, MXFP4, dequant

QB = 64                               # contraction block of the INT8 operands
F32 = np.float32


def q8_encode(x: np.ndarray):
    """INT8 codes of a set of fp32-exact values sharing one scale -> (codes int32, scale)."""
    x32 = np.asarray(x, dtype=np.float32)
    a = F32(np.max(np.abs(x32))) if x32.size else F32(0)
    if a == 0:
        return np.zeros(x32.shape, np.int32), 0.0
    s = F32(a / F32(127))
    r = F32(F32(127) / a)
    u = (x32 * r).astype(np.float32)
    return np.clip(np.rint(u), -127, 127).astype(np.int32), float(s)


def q8_rows(X: np.ndarray):
    """INT8 encoding of X [R, C] (C a multiple of QB) with one scale per (row, block of QB
    columns), as q8_encode on each such set, vectorised. Returns (codes int32 [R, C],
    scales float64 [R, C/QB], u float32 [R, C]: the scaled values before rounding)."""
    X = np.asarray(X, dtype=np.float32)
    R, C = X.shape
    Xb = X.reshape(R, C // QB, QB)
    a = np.max(np.abs(Xb), axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(a > 0, (a / F32(127)).astype(np.float32), F32(0)).astype(np.float32)
        r = np.where(a > 0, (F32(127) / a).astype(np.float32), F32(0)).astype(np.float32)
    u = (Xb * r[:, :, None]).astype(np.float32)
    codes = np.clip(np.rint(u), -127, 127).astype(np.int32)
    return codes.reshape(R, C), s.astype(np.float64), u.reshape(R, C)


def q8_tokens(X: np.ndarray):
    """Token-major operand X [N, D] (Q^, K^ or dO): one scale per (channel, 64-token block).
    Returns (codes [D, Np] int32, scales [D, Np/QB]), Np = ceil(N/QB)*QB, zero past N."""
    N, D = X.shape
    Np = -(-N // QB) * QB
    Xt = np.zeros((D, Np), np.float32)
    Xt[:, :N] = np.asarray(X, np.float32).T
    codes, s, _ = q8_rows(Xt)
    return codes, s


def _int8_mm(At, sA, Bt, sB):
    """sum over blocks b of (sA[:, b] sB[:, b]^T) * (At[:, b] @ Bt[:, b]^T): At [R, Np] and
    Bt [C, Np] INT8 codes with per-(row, block) scales sA [R, nb], sB [C, nb]; exact integer
    products, float64 sums."""
    R, Np = At.shape
    out = np.zeros((R, Bt.shape[0]))
    for b in range(Np // QB):
        rs = slice(b * QB, (b + 1) * QB)
        out += np.outer(sA[:, b], sB[:, b]) * (At[:, rs].astype(np.float64) @ Bt[:, rs].T.astype(np.float64))
    return out


def _near_half(u: np.ndarray, e: np.ndarray) -> np.ndarray:
    """True where u lies within e of a rounding boundary k + 1/2."""
    return np.abs(np.abs(u - np.floor(u)) - 0.5) <= e


def _ambiguous(eX, u, sc):
    """Codes whose scaled value u lies within its float32 error of a half-integer. eX: the
    error bound of each encoded value; sc: the per-(row, block) scales."""
    R, C = eX.shape
    a = 127.0 * np.repeat(sc, QB, axis=1)            # block maximum of each element
    with np.errstate(divide="ignore", invalid="ignore"):
        ra = np.where(a > 0, 127.0 / a, 0.0)
        emax = np.repeat(np.max(eX.reshape(R, C // QB, QB), axis=2), QB, axis=1)
        e = eX * ra + np.abs(u) * emax * ra / 127.0 + 2.0 ** -21 * np.abs(u)
    return _near_half(u.astype(np.float64), e) & (a > 0)


def _el(sc):
    return np.repeat(sc, QB, axis=1)


def _slack_mag(X, eX, codes, sc, u, wB):
    """Slack and magnitude of an INT8 matmul's outputs. X [R, C]: the encoded operand's values
    (rows are the scale owners), eX: their float32 error bounds, codes / sc / u: its encoding,
    wB [C, D]: |B codes| times B's scales. Per (row, block), with a the block maximum and emax
    the largest error in the block:
      - rel = emax / a > 1/254: the kernel's scale may differ enough to move a code by half a
        step or more (the maximum is near rounding-noise level, e.g. a causal row whose dS
        cancels to zero), so each element contributes up to 2 (|x| + e + (a + emax) / 127) |B|;
      - otherwise a code moves by at most |u| rel <= half a step, i.e. only a code within
        its error (which includes |u| rel) of a half-integer may move, by one step; and the
        kernel's scale may differ by rel, which moves every term by rel of itself.
    Returns (slack [R, D], mag [R, D], number of ambiguous codes, number of noise-level blocks)."""
    R, C = X.shape
    a = 127.0 * _el(sc)
    emax = np.repeat(np.max(eX.reshape(R, C // QB, QB), axis=2), QB, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(a > 0, emax / a, np.where(emax > 0, np.inf, 0.0))
    noisy = rel > 1.0 / 254.0
    amb = _ambiguous(eX, u, sc) & ~noisy
    term = np.abs(codes) * _el(sc)
    w = np.where(noisy, 2.0 * (np.abs(X) + eX + (a + emax) / 127.0), amb * _el(sc) + np.where(noisy, 0.0, rel) * term)
    return w @ wB, term @ wB, int(amb.sum()), int(noisy.sum()) // QB


def _block(Qp, Kp, Vp, Op, dOp, lsep, N, D, c, causal, I, J, want_bounds):
    """S, P, dP, dS of query rows I and key columns J (index arrays over the padded tokens), and
    with want_bounds the float32 error bounds of P and dS: dot products of D exact terms
    (error <= D 2^-24 sum|terms|), exp of an argument near |c S| + |lse|, a factor 4 of margin."""
    i = I[:, None]
    j = J[None, :]
    vis = (i < N) & (j < N)
    if causal:
        vis &= j <= i
    S = Qp[I] @ Kp[J].T
    with np.errstate(over="ignore"):
        P = np.where(vis, np.exp(np.where(vis, c * S - lsep[I][:, None], -np.inf)), 0.0)
    dP = dOp[I] @ Vp[J].T
    Dl = np.sum(dOp[I] * Op[I], axis=1)
    dS = P * (dP - Dl[:, None])
    if not want_bounds:
        return P, dS, None, None
    g = D * 2.0 ** -24
    aQ, aK, aV, aO, adO = np.abs(Qp[I]), np.abs(Kp[J]), np.abs(Vp[J]), np.abs(Op[I]), np.abs(dOp[I])
    relP = 4.0 * (c * g * (aQ @ aK.T) + 2.0 ** -22 * (np.abs(c * S) + np.abs(lsep[I][:, None]) + 1.0) + 2.0 ** -21)
    eP = np.where(vis, P * relP, 0.0)
    edS = 4.0 * (P * (g * (adO @ aV.T) + g * np.sum(adO * aO, axis=1)[:, None]) + np.abs(dS) * relP)
    edS = np.where(vis, edS + 2.0 ** -22 * np.abs(dS), 0.0)
    return P, dS, eP, edS


def _head(Qh, Kh, V, O, dO, lse, N, D, c, causal, quantize, want_bounds, keys=None, queries=None):
    """One head. keys / queries: None for all, else the token indices whose dK, dV (keys) and dQ
    (queries) are wanted. A key's gradients need only its column of S (over all queries) and a
    query's only its row, and every INT8 scale of P and dS belongs to one row of its operand, so
    selected gradients come out exactly as in the full computation (their slack and mag up to
    float64 summation order)."""
    Np = -(-N // QB) * QB
    pad = Np - N

    def padr(X):
        return np.pad(X, ((0, pad), (0, 0))) if pad else X

    Qp, Kp, Vp, Op, dOp = (padr(X) for X in (Qh, Kh, V, O, dO))
    lsep = np.pad(lse, (0, pad))
    every = np.arange(Np)
    J = every if keys is None else np.asarray(keys, np.int64)
    I = every if queries is None else np.asarray(queries, np.int64)
    if not quantize:
        Pc, dSc, _, _ = _block(Qp, Kp, Vp, Op, dOp, lsep, N, D, c, causal, every, J, False)
        _, dSr, _, _ = _block(Qp, Kp, Vp, Op, dOp, lsep, N, D, c, causal, I, every, False)
        dV = Pc.T @ dOp
        dK = c * (dSc.T @ Qp)
        dQ = c * (dSr @ Kp)
        if keys is None and queries is None:
            return dQ[:N], dK[:N], dV[:N], None
        return dQ, dK, dV, None

    Qt, sQ = q8_tokens(Qh)                       # [D, Np], per (channel, query block)
    Kt, sK = q8_tokens(Kh)
    dOt, sdO = q8_tokens(dO)
    # keys J: columns of S over every query
    Pc, dSc, ePc, edSc = _block(Qp, Kp, Vp, Op, dOp, lsep, N, D, c, causal, every, J, want_bounds)
    Pk, sPk, uP = q8_rows(Pc.T)                  # P^T [keys, queries], per (key, query block)
    dSk, sSk, uk = q8_rows(dSc.T)                # dS^T [keys, queries], per (key, query block)
    dV = _int8_mm(Pk, sPk, dOt, sdO)
    dK = c * _int8_mm(dSk, sSk, Qt, sQ)
    # queries I: rows of S over every key
    _, dSr, _, edSr = _block(Qp, Kp, Vp, Op, dOp, lsep, N, D, c, causal, I, every, want_bounds)
    dSq, sSq, uq = q8_rows(dSr)                  # dS [queries, keys], per (query, key block)
    dQ = c * _int8_mm(dSq, sSq, Kt, sK)
    bounds = None
    if want_bounds:
        wdO = (np.abs(dOt) * _el(sdO)).T                  # [Np, D]
        wQ = (np.abs(Qt) * _el(sQ)).T
        wK = (np.abs(Kt) * _el(sK)).T
        sV, mV, aV, nV = _slack_mag(Pc.T, ePc.T, Pk, sPk, uP, wdO)          # rows: keys
        sK_, mK, aK, nK = _slack_mag(dSc.T, edSc.T, dSk, sSk, uk, wQ)       # rows: keys
        sQ_, mQ, aQ, nQ = _slack_mag(dSr, edSr, dSq, sSq, uq, wK)           # rows: queries
        bounds = dict(slack=[c * sQ_, c * sK_, sV], mag=[c * mQ, c * mK, mV],
                      n_amb=(aQ, aK, aV), n_noisy_blocks=(nQ, nK, nV))
    if keys is None and queries is None:
        if bounds is not None:
            bounds["slack"] = tuple(x[:N] for x in bounds["slack"])
            bounds["mag"] = tuple(x[:N] for x in bounds["mag"])
        return dQ[:N], dK[:N], dV[:N], bounds
    return dQ, dK, dV, bounds


def attn_bwd(fmt, q, k, v, o, do, lse, causal=False, sm_scale=0.0, heads=None, quantize=True,
             want_bounds=False):
    """Gradients of the quantised attention (reading R16 in this module's docstring).

    q, k: (codes, scales) of the forward's Q and K (``oracle.quant``; MX4_PV8 uses MXFP4 Q/K);
    v, o, do: [B,H,N,D] (float16 values); lse: [B,H,N] (the forward stores float32 values).
    heads: None for all, or a list of (b, h) to compute (the others are returned as zeros).
    quantize=False: the same gradients with every matmul in float64 (no INT8 step).
    Returns (dq, dk, dv) float64 [B,H,N,D]; with want_bounds also a dict of per-element
    'slack' and 'mag' tuples (dq, dk, dv), the number of ambiguous codes 'n_amb' and of
    (row, block) encodings whose maximum is at rounding-noise level 'n_noisy_blocks'."""
    fq = MXFP4 if fmt == MX4_PV8 else fmt
    B, H, N, D = v.shape
    c = float(np.float32(1.0 / np.sqrt(D))) if sm_scale <= 0 else float(np.float32(sm_scale))
    out = [np.zeros((B, H, N, D)) for _ in range(3)]
    sl = [np.zeros((B, H, N, D)) for _ in range(3)] if want_bounds else None
    mg = [np.zeros((B, H, N, D)) for _ in range(3)] if want_bounds else None
    namb = [0, 0, 0]
    nnoisy = [0, 0, 0]
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        Qh = dequant(fq, q[0][b, h], q[1][b, h])
        Kh = dequant(fq, k[0][b, h], k[1][b, h])
        V, O, dO = (np.asarray(X[b, h], np.float64) for X in (v, o, do))
        L = np.asarray(lse[b, h], np.float64)
        r = _head(Qh, Kh, V, O, dO, L, N, D, c, causal, quantize, want_bounds)
        for t in range(3):
            out[t][b, h] = r[t]
        if want_bounds:
            for t in range(3):
                sl[t][b, h] = r[3]["slack"][t]
                mg[t][b, h] = r[3]["mag"][t]
                namb[t] += r[3]["n_amb"][t]
                nnoisy[t] += r[3]["n_noisy_blocks"][t]
    if want_bounds:
        return tuple(out), dict(slack=tuple(sl), mag=tuple(mg), n_amb=tuple(namb), n_noisy_blocks=tuple(nnoisy))
    return tuple(out)


def attn_bwd_sampled(fmt, q, k, v, o, do, lse, head, keys, queries, causal=False, sm_scale=0.0,
                     want_bounds=True):
    """The same gradients for one head (b, h) at selected tokens, without forming N x N arrays:
    dK and dV of `keys` and dQ of `queries` (token indices < N). Returns (dq [len(queries), D],
    dk [len(keys), D], dv [len(keys), D]) and, with want_bounds, the matching slack / mag."""
    fq = MXFP4 if fmt == MX4_PV8 else fmt
    B, H, N, D = v.shape
    b, h = head
    c = float(np.float32(1.0 / np.sqrt(D))) if sm_scale <= 0 else float(np.float32(sm_scale))
    Qh = dequant(fq, q[0][b, h], q[1][b, h])
    Kh = dequant(fq, k[0][b, h], k[1][b, h])
    V, O, dO = (np.asarray(X[b, h], np.float64) for X in (v, o, do))
    L = np.asarray(lse[b, h], np.float64)
    r = _head(Qh, Kh, V, O, dO, L, N, D, c, causal, True, want_bounds, keys=keys, queries=queries)
    if want_bounds:
        return r[:3], dict(slack=tuple(r[3]["slack"]), mag=tuple(r[3]["mag"]), n_amb=r[3]["n_amb"],
                           n_noisy_blocks=r[3]["n_noisy_blocks"])
    return r[:3]
