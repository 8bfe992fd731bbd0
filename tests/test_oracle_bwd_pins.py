"""Planted pins of the backward oracle's per-element bound (|gpu - oracle| <= slack + 1e-4 mag).

The bound's slack has three parts (oracle/bwd.py, _slack_mag and _ambiguous):
  - a P or dS code whose scaled value lies within its float32 error of a half-integer may be
    rounded either way: the slack adds the effect of the other choice;
  - the kernel's block scale may differ from the oracle's by the block maximum's own error;
  - a block whose maximum is at its own rounding-noise level can take any codes: every element
    adds 2 (|x| + e + (a + emax)/127) |B|.

Each part is pinned here by inputs that put it to work exactly, on one 64-token block (N = 64,
D = 128). Q = 0 or K = 0 makes S = 0, so P = exp(-lse) row by row and dS = P (dP - D) come out
exact from small fp16 values; the other operand of the planted gradient is +-1, so every output
element sees the same one-code effect:
  - a tie u = k + 1/2 planted in P (for dV), in dS^T (for dK) and in dS (for dQ): rounding the
    tie the other way must move the gradient by no more than the slack, and by at least 95% of
    it (so an inflated slack fails);
  - the same inputs moved off the tie: no ambiguous code, and the slack is the scale term alone,
    under 2% of one code step's effect;
  - dS = 0 exactly (dP = D): every dS block is at noise level, and an adversarial kernel whose
    dS values sit at the edge of their error bound, signed to add up, must stay within the slack
    and reach at least 40% of it (the term's factor 2 is its only margin).
"""
from contextlib import contextmanager

import numpy as np

import oracle as orc
from oracle import bwd

N, D = 64, 128
FMT = orc.NVFP4


@contextmanager
def ties_rounded_the_other_way():
    """Every INT8 encoding of an N x N operand (P^T, dS^T, dS) rounds its exact ties u = k + 1/2
    away from the even code; the token-major encodings of Q^, K^ and dO ([D, N]) are untouched
    (the kernel computes those from identical inputs, bit for bit)."""
    orig = bwd.q8_rows

    def flipped(X):
        codes, s, u = orig(X)
        if X.shape == (N, N):
            uu = u.astype(np.float64)
            tie = (uu - np.floor(uu)) == 0.5
            codes = np.where(tie, np.rint(2.0 * uu).astype(np.int64) - codes, codes).astype(np.int32)
        return codes, s, u

    bwd.q8_rows = flipped
    try:
        yield
    finally:
        bwd.q8_rows = orig


def _signs(rng):
    return rng.choice(np.array([-1.0, 1.0], np.float16), size=(1, 1, N, D))


def _qk(zero_q, rng):
    """Q^ (or K^) of +-1 inputs: NVFP4 encodes every one as +-6 * 0.171875 = +-1.03125."""
    x = _signs(rng)
    z = np.zeros((1, 1, N, D), np.float16)
    q, k = (z, x) if zero_q else (x, z)
    return orc.quant(orc.ROLE_Q, FMT, q), orc.quant(orc.ROLE_K, FMT, k)


def _e0(vals):
    """[1,1,N,D] fp16 with column 0 = vals, zeros elsewhere."""
    a = np.zeros((1, 1, N, D), np.float16)
    a[0, 0, :, 0] = vals
    return a


def _run(Q, K, v, o, do, lse):
    return bwd.attn_bwd(FMT, Q, K, v, o, do, lse, want_bounds=True)


def _pinned_flip(t, Q, K, v, o, do, lse, n_planted):
    """Gradient t (0 dq, 1 dk, 2 dv): the planted ties are the only ambiguous codes, and the
    other rounding moves the gradient within the slack and by at least 95% of it."""
    g, bd = _run(Q, K, v, o, do, lse)
    assert bd["n_amb"][t] == n_planted and bd["n_noisy_blocks"][t] == 0, (bd["n_amb"], bd["n_noisy_blocks"])
    with ties_rounded_the_other_way():
        g2 = bwd.attn_bwd(FMT, Q, K, v, o, do, lse)
    eff = np.abs(g2[t] - g[t])
    sl = bd["slack"][t]
    moved = eff > 0
    assert moved.sum() > 0.5 * moved.size, "the planted ties must move most elements"
    assert np.all(eff <= sl * (1 + 1e-12)), float(np.max(eff / np.where(sl > 0, sl, 1.0)))
    assert np.min(eff[moved] / sl[moved]) >= 0.95, float(np.min(eff[moved] / sl[moved]))
    for u in range(3):
        if u != t:
            assert np.array_equal(g2[u], g[u])
    return g, bd


def _off_tie(t, Q, K, v, o, do, lse, step_effect):
    """The same case off the tie: no ambiguous code; the slack is the scale term alone, under 2%
    of one code step's effect."""
    g, bd = _run(Q, K, v, o, do, lse)
    assert bd["n_amb"][t] == 0 and bd["n_noisy_blocks"][t] == 0, (bd["n_amb"], bd["n_noisy_blocks"])
    sl = bd["slack"][t]
    big = step_effect > 0
    assert np.all(sl[big] <= 0.02 * step_effect[big]), float(np.max(sl[big] / step_effect[big]))


def test_tie_in_p_for_dv():
    """K = 0: P[i, j] = exp(-lse_i). lse_0 = 0 gives the block maximum 1 and lse_1 = fl32(ln 2)
    gives P = 0.5 in float32, so u = 0.5 * 127 = 63.5 for every key; the other queries have
    lse = 200 (P = 0 in float32). dO = +-1."""
    rng = np.random.default_rng(1)
    Q, K = _qk(zero_q=False, rng=rng)
    v, o = (rng.standard_normal((1, 1, N, D)).astype(np.float16) for _ in range(2))
    do = _signs(rng)
    lse = np.full((1, 1, N), 200.0, np.float32)
    lse[0, 0, 0] = 0.0
    lse[0, 0, 1] = np.float32(np.log(2.0))
    _pinned_flip(2, Q, K, v, o, do, lse, n_planted=N)
    # off the tie: P_1 = 0.375 (u = 47.625); one code step moves dV[j, :] by |dO[1, :]| / 127
    lse[0, 0, 1] = np.float32(-np.log(0.375))
    step = np.full((1, 1, N, D), 1.0 / 127.0)
    _off_tie(2, Q, K, v, o, do, lse, step)


def test_tie_in_ds_transposed_for_dk():
    """K = 0, lse = 0: P = 1. dO = V = e0 (column 0 = 1) gives dP = 1, and O[:, 0] = o gives
    D_i = o_i, so dS[i, j] = 1 - o_i: o = (0, 0.5, 1, ...) puts u = 63.5 at query 1 of every
    key; every query row of dS is constant (no tie for dQ). Q = +-1."""
    rng = np.random.default_rng(2)
    Q, K = _qk(zero_q=False, rng=rng)
    ov = np.full(N, 1.0)
    ov[0], ov[1] = 0.0, 0.5
    v, o, do = _e0(1.0), _e0(ov), _e0(1.0)
    lse = np.zeros((1, 1, N), np.float32)
    _pinned_flip(1, Q, K, v, o, do, lse, n_planted=N)
    # off the tie: o_1 = 0.625 (u = 47.625); one code step moves dK[j, :] by c * |Q^[1, :]| / 127
    ov[1] = 0.625
    c = float(np.float32(1.0 / np.sqrt(D)))
    qh = orc.dequant(FMT, *Q)[0, 0]
    step = c * np.abs(qh[1])[None, :] / 127.0 * np.ones((N, 1))
    _off_tie(1, Q, K, v, _e0(ov), do, lse, step[None, None])


def test_tie_in_ds_for_dq():
    """Q = 0, lse = 0: P = 1. dO = e0, V[:, 0] = v, O = 0: dS[i, j] = v_j, with
    v = (1, 0.5, 0, ...) a tie u = 63.5 at key 1 of every query; every key column of dS is
    constant (no tie for dK). K = +-1."""
    rng = np.random.default_rng(3)
    Q, K = _qk(zero_q=True, rng=rng)
    vv = np.full(N, 0.0)
    vv[0], vv[1] = 1.0, 0.5
    o = np.zeros((1, 1, N, D), np.float16)
    lse = np.zeros((1, 1, N), np.float32)
    _pinned_flip(0, Q, K, _e0(vv), o, _e0(1.0), lse, n_planted=N)
    vv[1] = 0.375
    c = float(np.float32(1.0 / np.sqrt(D)))
    kh = orc.dequant(FMT, *K)[0, 0]
    step = c * np.abs(kh[1])[None, :] / 127.0 * np.ones((N, 1))
    _off_tie(0, Q, K, _e0(vv), o, _e0(1.0), lse, step[None, None])


def _adversarial_noise(t, Q, K, v, o, do, lse, sign_rows):
    """dS = 0 exactly: every dS block is at noise level. The adversarial kernel's dS values are
    their error bound edS with the sign of the other operand in column 0 (sign_rows: [N] signs
    over the contracted index), so that their effect on column 0 adds up."""
    g, bd = _run(Q, K, v, o, do, lse)
    assert bd["n_noisy_blocks"][t] > 0, bd
    orig = bwd._block

    def adversarial(Qp, Kp, Vp, Op, dOp, lsep, N_, D_, c, causal, I, J, want_bounds):
        P, dS, eP, edS = orig(Qp, Kp, Vp, Op, dOp, lsep, N_, D_, c, causal, I, J, True)
        assert np.all(dS == 0)
        if t == 1:    # dK: contracted over queries I (rows of dS)
            adv = edS * sign_rows[I][:, None]
        else:         # dQ: contracted over keys J (columns of dS)
            adv = edS * sign_rows[J][None, :]
        return (P, adv, eP, edS) if want_bounds else (P, adv, None, None)

    bwd._block = adversarial
    try:
        g2 = bwd.attn_bwd(FMT, Q, K, v, o, do, lse)
    finally:
        bwd._block = orig
    eff = np.abs(g2[t] - g[t])[0, 0, :, 0]
    sl = bd["slack"][t][0, 0, :, 0]
    assert np.all(eff <= sl), float(np.max(eff / sl))
    assert np.min(eff / sl) >= 0.4, float(np.min(eff / sl))


def test_noise_level_ds_blocks_for_dk():
    """K = 0, lse = 0, dO = V = O = e0: dP = D = 1, so dS = 0 exactly for every (query, key)."""
    rng = np.random.default_rng(4)
    Q, K = _qk(zero_q=False, rng=rng)
    qh = orc.dequant(FMT, *Q)[0, 0]
    sgn = np.sign(qh[:, 0])
    sgn[sgn == 0] = 1.0
    _adversarial_noise(1, Q, K, _e0(1.0), _e0(1.0), _e0(1.0), np.zeros((1, 1, N), np.float32), sgn)


def test_noise_level_ds_blocks_for_dq():
    """Q = 0, lse = 0, dO = V = O = e0: dS = 0 exactly; the adversary signs follow K^'s column 0."""
    rng = np.random.default_rng(5)
    Q, K = _qk(zero_q=True, rng=rng)
    kh = orc.dequant(FMT, *K)[0, 0]
    sgn = np.sign(kh[:, 0])
    sgn[sgn == 0] = 1.0
    _adversarial_noise(0, Q, K, _e0(1.0), _e0(1.0), _e0(1.0), np.zeros((1, 1, N), np.float32), sgn)
