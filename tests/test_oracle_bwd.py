"""Pins of the backward oracle (oracle/bwd.py) against things other than itself.

- INT8 encoder: hand-computed codes (ties to even, the block maximum at +-127, all-zero blocks)
  and the rounding bound |code * scale - x| <= scale / 2 on random data.
- Unquantised mode against torch.autograd in float64 on the same dequantised Q^, K^ and fp16 V
  (gradients of sum(O * dO) for O = softmax(c Q^ K^T) V), causal or not, ragged N.
- Closed forms that any attention gradient satisfies with the exact O and lse: the key
  gradients sum to zero (softmax is invariant to adding one vector to every key) and the value
  gradients sum to the summed output gradient (each row of P sums to one).
- INT8 mode on one-hot attention, where every encoding the method makes is lossless or
  multiplies a value below 1e-30: dV is the sum of the dO rows that pick each key, dQ = dK = 0.
- INT8 granularity: one outlier in dO changes no dV column but its own (scales per channel and
  64-token block), and the INT8 gradients stay within a few percent of the unquantised ones.
- The tolerance model the GPU tests use: a float32 twin that rounds the way a kernel does
  (float32 S, exp2, dP, D, dS; integer products; float32 sums) stays within the oracle's slack
  plus 1e-4 of the magnitudes.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from oracle import bwd
from bit_attention_amd import synth


def q8_reference(x):
    """Codes the plain way: x / scale in float64, rounded half to even."""
    a = np.float32(np.max(np.abs(x)))
    s = np.float32(a / np.float32(127))
    return np.rint(np.asarray(x, np.float64) / float(s)), float(s)


def test_q8_encode_hand_cases():
    x = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.0, -127.0, 126.5], np.float32)
    codes, s = bwd.q8_encode(x)
    assert s == 1.0
    assert codes.tolist() == [127, 2, 4, -2, -4, 0, 2, 0, -127, 126]
    codes, s = bwd.q8_encode(np.zeros(64, np.float32))
    assert s == 0.0 and not codes.any()
    # a block whose maximum is negative: it still maps to -127
    codes, s = bwd.q8_encode(np.array([-6.0, 3.0, 1.0], np.float32))
    assert codes.tolist() == [-127, 64, 21] and s == float(np.float32(6.0 / 127.0))


def test_q8_rows_rounding_bound():
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((40, 256)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    X[3, 64:128] = 0.0
    codes, s, _ = bwd.q8_rows(X)
    assert s.shape == (40, 4) and np.all(s[3, 1] == 0) and not codes[3, 64:128].any()
    for r in range(40):
        for b in range(4):
            blk = X[r, 64 * b:64 * (b + 1)]
            cb = codes[r, 64 * b:64 * (b + 1)]
            if s[r, b] == 0:
                continue
            assert np.abs(cb).max() == 127 and np.abs(cb[np.argmax(np.abs(blk))]) == 127
            err = np.abs(cb * s[r, b] - blk.astype(np.float64))
            assert np.all(err <= s[r, b] * (0.5 + 1e-5))
            ref, sr = q8_reference(blk)
            assert sr == s[r, b]
            far = np.abs(np.abs(blk / sr - np.floor(blk / sr)) - 0.5) > 1e-4
            assert np.array_equal(cb[far], ref[far])


def _setup(fmt, N, D, causal, H=2):
    q, k, v = synth.make_qkv(1, N=N, D=D, H=H)
    do = synth.make_do(1, N=N, D=D, H=H)
    fq = orc.MXFP4 if fmt == orc.MX4_PV8 else fmt
    Q = orc.quant(orc.ROLE_Q, fq, q)
    K = orc.quant(orc.ROLE_K, fq, k)
    return q, k, v, do, Q, K


def _torch_grads(Qh, Kh, V, dO, c, causal):
    Qt = torch.tensor(Qh, dtype=torch.float64, requires_grad=True)
    Kt = torch.tensor(Kh, dtype=torch.float64, requires_grad=True)
    Vt = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    S = c * (Qt @ Kt.transpose(-1, -2))
    if causal:
        N = S.shape[-1]
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(S, dim=-1)
    O = torch.softmax(S, dim=-1) @ Vt
    (O * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return (Qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy(), O.detach().numpy(), lse.detach().numpy())


@pytest.mark.parametrize("fmt,N,D,causal", [(orc.NVFP4, 200, 64, False), (orc.NVFP4, 200, 64, True),
                                            (orc.MXFP4, 130, 128, True), (orc.MXFP4, 64, 64, False)])
def test_unquantised_mode_matches_autograd(fmt, N, D, causal):
    q, k, v, do, Q, K = _setup(fmt, N, D, causal)
    Qh = orc.dequant(fmt, *Q)
    Kh = orc.dequant(fmt, *K)
    c = float(np.float32(1.0 / np.sqrt(D)))
    gq, gk, gv, O, lse = _torch_grads(Qh, Kh, v.astype(np.float64), do.astype(np.float64), c, causal)
    dq, dk, dv = bwd.attn_bwd(fmt, Q, K, v, O, do, lse, causal=causal, quantize=False)
    for got, ref in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-11 * np.abs(ref).max())


@pytest.mark.parametrize("causal", [False, True])
def test_unquantised_mode_closed_forms(causal):
    fmt, N, D = orc.NVFP4, 190, 64
    q, k, v, do, Q, K = _setup(fmt, N, D, causal)
    Qh = orc.dequant(fmt, *Q)
    Kh = orc.dequant(fmt, *K)
    c = float(np.float32(1.0 / np.sqrt(D)))
    _, _, _, O, lse = _torch_grads(Qh, Kh, v.astype(np.float64), do.astype(np.float64), c, causal)
    dq, dk, dv = bwd.attn_bwd(fmt, Q, K, v, O, do, lse, causal=causal, quantize=False)
    scale = np.abs(dk).max()
    assert np.abs(dk.sum(axis=2)).max() <= 1e-11 * scale * N
    np.testing.assert_allclose(dv.sum(axis=2), do.astype(np.float64).sum(axis=2), rtol=1e-11, atol=1e-11)
    assert np.abs(dq).max() > 0.01 and scale > 0.01


def _one_hot_case(fmt, causal):
    N = D = 64
    t = (np.arange(N) // 2) if causal else (5 * np.arange(N) + 3) % N
    q = np.zeros((1, 1, N, D), np.float16)
    k = np.zeros((1, 1, N, D), np.float16)
    q[0, 0, np.arange(N), t] = 24.0
    k[0, 0, np.arange(N), np.arange(N)] = 24.0
    v = synth.make_qkv(1, N=N, D=D, H=1)[2]
    rng = np.random.default_rng(11)
    kk = rng.integers(-126, 127, (N, D))
    kk[0, :] = 127                                   # every (channel, 64-token block) reaches 127
    do = (kk / 128.0).astype(np.float16)[None, None]
    Q = orc.quant(orc.ROLE_Q, fmt, q)
    K = orc.quant(orc.ROLE_K, fmt, k)
    O = v[:, :, t, :]                                # the row picks key t(i) alone
    lse = np.full((1, 1, N), 72.0)                   # c S = 576 / 8 on the picked key, 0 elsewhere
    return t, v, do, Q, K, O, lse


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4])
@pytest.mark.parametrize("causal", [False, True])
def test_int8_one_hot_attention(fmt, causal):
    t, v, do, Q, K, O, lse = _one_hot_case(fmt, causal)
    assert np.array_equal(orc.dequant(fmt, *Q)[0, 0][np.arange(64), t], np.full(64, 24.0))
    want = np.zeros((64, 64))
    np.add.at(want, t, do[0, 0].astype(np.float64))
    for quantize in (True, False):
        dq, dk, dv = bwd.attn_bwd(fmt, Q, K, v, O, do, lse, causal=causal, quantize=quantize)
        np.testing.assert_allclose(dv[0, 0], want, rtol=1e-6, atol=1e-12)
        assert np.abs(dq).max() < 1e-9 and np.abs(dk).max() < 1e-9


def test_int8_scale_granularity_and_error():
    fmt, N, D = orc.NVFP4, 256, 64
    q, k, v, do, Q, K = _setup(fmt, N, D, False, H=1)
    o, lse = orc.attn_fwd(fmt, Q, K, orc.quant(orc.ROLE_V, fmt, v), q.shape, want_lse=True)
    o = o.astype(np.float16)
    lse = lse.reshape(1, 1, N)
    dq, dk, dv = bwd.attn_bwd(fmt, Q, K, v, o, do, lse)
    eq, ek, ev = bwd.attn_bwd(fmt, Q, K, v, o, do, lse, quantize=False)
    for got, ref in ((dq, eq), (dk, ek), (dv, ev)):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert 1e-4 < rel < 0.03, rel
    do2 = do.copy()
    do2[0, 0, 70, 9] = 60.0
    dv2 = bwd.attn_bwd(fmt, Q, K, v, o, do2, lse)[2]
    others = np.arange(D) != 9
    assert np.array_equal(dv2[..., others], dv[..., others])
    assert not np.array_equal(dv2[..., 9], dv[..., 9])


def _f32_twin(fmt, Q, K, v, o, do, lse, causal, c):
    """The INT8 backward the way a kernel rounds it: float32 S, exp2, dP, D and dS, the INT8
    encodings of the definition, integer block products, float32 sums."""
    f = np.float32
    Qh = orc.dequant(fmt, *Q)[0, 0].astype(f)
    Kh = orc.dequant(fmt, *K)[0, 0].astype(f)
    V, O, dO = (x[0, 0].astype(f) for x in (v, o, do))
    N, D = V.shape
    Np = -(-N // 64) * 64

    def pad(X):
        return np.pad(X, ((0, Np - N), (0, 0)))

    Qh, Kh, V, O, dO = (pad(X) for X in (Qh, Kh, V, O, dO))
    L = np.pad(lse[0, 0].astype(f), (0, Np - N))
    i, j = np.arange(Np)[:, None], np.arange(Np)[None, :]
    vis = (i < N) & (j < N) & ((j <= i) if causal else True)
    S = (Qh @ Kh.T).astype(f)
    l2e = f(1.4426950408889634)
    P = np.where(vis, np.exp2((S * f(c * l2e) - L[:, None] * l2e).astype(f)), f(0)).astype(f)
    dP = (dO @ V.T).astype(f)
    Dl = np.sum(dO * O, axis=1, dtype=f)
    dS = (P * (dP - Dl[:, None])).astype(f)

    def rows(X):
        return bwd.q8_rows(X)[:2]

    def tok(X):
        return rows(np.ascontiguousarray(X.T))

    def mm(A, sA, Bm, sB):
        out = np.zeros((A.shape[0], Bm.shape[0]), f)
        for b in range(Np // 64):
            rs = slice(64 * b, 64 * b + 64)
            acc = (A[:, rs].astype(np.int64) @ Bm[:, rs].T.astype(np.int64)).astype(f)
            out = (out + acc * np.outer(sA[:, b], sB[:, b]).astype(f)).astype(f)
        return out

    Qt, sQ = tok(Qh)
    Kt, sK = tok(Kh)
    dOt, sdO = tok(dO)
    Pk, sPk = rows(P.T)
    dSk, sSk = rows(dS.T)
    dSq, sSq = rows(dS)
    return (f(c) * mm(dSq, sSq, Kt, sK))[:N], (f(c) * mm(dSk, sSk, Qt, sQ))[:N], mm(Pk, sPk, dOt, sdO)[:N]


@pytest.mark.parametrize("fmt,N,D,causal", [(orc.NVFP4, 200, 64, False), (orc.MXFP4, 160, 128, True)])
def test_float32_twin_within_slack(fmt, N, D, causal):
    q, k, v, do, Q, K = _setup(fmt, N, D, causal, H=1)
    o, lse = orc.attn_fwd(fmt, Q, K, orc.quant(orc.ROLE_V, fmt, v), q.shape, causal=causal, want_lse=True)
    o = o.astype(np.float16)
    lse = lse.astype(np.float32).reshape(1, 1, N)
    c = float(np.float32(1.0 / np.sqrt(D)))
    (dq, dk, dv), bd = bwd.attn_bwd(fmt, Q, K, v, o, do, lse, causal=causal, want_bounds=True)
    twin = _f32_twin(fmt, Q, K, v, o, do, lse, causal, c)
    for t, (got, ref) in enumerate(zip(twin, (dq[0, 0], dk[0, 0], dv[0, 0]))):
        bound = bd["slack"][t][0, 0] + 1e-4 * bd["mag"][t][0, 0] + 1e-30
        assert np.all(np.abs(got - ref) <= bound), (t, np.max(np.abs(got - ref) / bound))
    assert all(n < 0.1 * N * N for n in bd["n_amb"])


@pytest.mark.parametrize("fmt,N,D,causal", [(orc.NVFP4, 200, 64, True), (orc.MXFP4, 130, 128, False)])
def test_sampled_mode_matches_full(fmt, N, D, causal):
    """Selected keys and queries (the mode used at sizes where N x N arrays do not fit) give the
    full computation's gradients bit for bit, and its bounds to float64 summation order."""
    q, k, v, do, Q, K = _setup(fmt, N, D, causal)
    o, lse = orc.attn_fwd(fmt, Q, K, orc.quant(orc.ROLE_V, fmt, v), q.shape, causal=causal, want_lse=True)
    o = o.astype(np.float16)
    lse = lse.astype(np.float32).reshape(q.shape[:3])
    full, bd = bwd.attn_bwd(fmt, Q, K, v, o, do, lse, causal=causal, want_bounds=True)
    keys = np.array([0, 5, 63, 64, N - 1])
    qs = np.array([1, 64, 100, N - 1])
    (sq, sk, sv), sb = bwd.attn_bwd_sampled(fmt, Q, K, v, o, do, lse, (0, 1), keys, qs, causal=causal)
    assert np.array_equal(sq, full[0][0, 1][qs])
    assert np.array_equal(sk, full[1][0, 1][keys]) and np.array_equal(sv, full[2][0, 1][keys])
    for t, rows in ((0, qs), (1, keys), (2, keys)):
        for part in ("slack", "mag"):
            ref = bd[part][t][0, 1][rows]
            np.testing.assert_allclose(sb[part][t], ref, rtol=1e-12, atol=1e-15 * max(1.0, np.abs(ref).max()))
