"""Pins of the oracle's slack: the per-row bound on how far a P rounding decision near its
boundary may move an output row (sage_oracle.c, "Slack").

Each case plants one decision exactly on a boundary, by choosing sm_scale so that the scaled score
difference of two keys puts the lower key's quotient on a tie. Q, K and V are exactly
representable, so the only rounding decisions are those of P. The pins:
  - on the boundary, the reported slack equals the output change that the flip causes, which is
    measured by nudging sm_scale by 1e-5 relative to each side of the tie (the flip is the only
    discontinuity; the continuous change is below 1e-4);
  - the same construction away from every boundary reports a slack of exactly 0;
  - the window grows with the scores' magnitude: a decision 0.1% from its boundary carries no
    slack at scores of order 1 and does at scores of order 10^4, where FP32 cannot resolve the
    difference of two scores to 0.1%.
Cases: NVFP4 E2M1 code tie, NVFP4 E4M3 block-scale tie, MXFP4 E2M1 code tie, MXFP4 E8M0 scale
boundary, and the Direct-P normaliser (a one-sided bound: it also covers the move of l)."""
import math

import numpy as np
import pytest

import oracle as orc

D = 64


def _qkv(N, kvals, vvals, big=False):
    """One head, two identical query rows: q[0] = 6, and (big) q[32] = 384; key j has k[0] =
    kvals[j] and (big) k[32] = 1536; V entries vvals[(key, channel)] = value. Every value is
    exactly representable in NVFP4 and MXFP4 (one nonzero per 32-channel block; 6 * 2^k)."""
    q = np.zeros((1, 1, 2, D), np.float16)
    q[..., 0] = 6.0
    k = np.zeros((1, 1, N, D), np.float16)
    k[0, 0, :, 0] = kvals
    if big:
        q[..., 32] = 384.0
        k[0, 0, :, 32] = 1536.0
    v = np.zeros((1, 1, N, D), np.float16)
    for (j, d), val in vvals.items():
        v[0, 0, j, d] = val
    return q, k, v


def _run(fmt, q, k, v, c, direct_p=False):
    N = k.shape[2]
    # the two query rows need the same keys: pad Q to N rows by repeating row 0
    qq = np.repeat(q[:, :, :1], N, axis=2)
    Q, K, V = (orc.quant(r, fmt, x) for x, r in ((qq, 0), (k, 1), (v, 2)))
    for x, (cod, sc), r in ((qq, Q, 0), (k, K, 1)):
        assert np.array_equal(orc.dequant(fmt, cod, sc), x.astype(np.float64)), "input not exact"
    out, slack = orc.attn_fwd(fmt, Q, K, V, (1, 1, N, D), sm_scale=c, rows=np.array([0]), want_slack=True,
                              direct_p=direct_p)
    return out[0].astype(np.float64), float(slack[0])


def _flip_check(fmt, q, k, v, c0, expect, direct_p=False, bound=None):
    """The outputs at c0 (1 -+ 1e-5) straddle the tie and differ by the flip's effect (expect,
    computed by hand), within the slack reported at c0 and at both nudged values. The slack equals
    expect (tight) or, when given, one of the hand-computed one-sided bounds."""
    o0, s0 = _run(fmt, q, k, v, c0, direct_p)
    lo, s_lo = _run(fmt, q, k, v, c0 * (1 - 1e-5), direct_p)
    hi, s_hi = _run(fmt, q, k, v, c0 * (1 + 1e-5), direct_p)
    flip = np.abs(lo - hi).max()
    assert flip == pytest.approx(expect, rel=1e-3), f"the planted decision did not flip ({flip} vs {expect})"
    for s in (s0, s_lo, s_hi):
        assert flip <= s + 1e-4, f"flip {flip} beyond slack {s}"
        if bound is None:
            assert s == pytest.approx(expect, rel=1e-5), f"slack {s}"
        else:
            assert min(abs(s / b - 1) for b in bound) < 1e-5, f"slack {s}, bounds {bound}"
    return flip, s0


def test_nvfp4_code_tie():
    """P2 quotient of key 1 = 6 exp(-18 c) = 2.5, the tie of E2M1 2 and 3 (block scale 448, fixed by
    the exact tile maximum). Flip: P-hat 896 <-> 1344, times V-hat 6 on channel 1, over 2688 l."""
    q, k, v = _qkv(2, [6.0, 3.0], {(0, 0): 6.0, (1, 1): 6.0})
    c0 = math.log(12 / 5) / 18
    l = 1 + 5 / 12
    _flip_check(orc.NVFP4, q, k, v, c0, 448 * 6 / (2688 * l))
    # 6 exp(-18 c) = 3.2: 9% from the nearest boundary (3.5), and the block scale is exact
    assert _run(orc.NVFP4, q, k, v, math.log(6 / 3.2) / 18)[1] == 0.0


def test_nvfp4_scale_tie():
    """Key 64 (slot 16, block 1) alone in its block: 448 E = 100, the midpoint of E4M3 96 and 104.
    The element saturates at code 6 under both scales, so the flip moves P-hat by 6 * 8 = 48.
    Keys 1..63 score 2304 below the maximum: E = 0 exactly, codes 0, scales 0."""
    kv = np.full(65, -384.0)
    kv[0], kv[64] = 6.0, 3.0
    q, k, v = _qkv(65, kv, {(0, 0): 6.0, (64, 1): 6.0})
    c0 = -math.log(100 / 448) / 18
    l = 1 + 100 / 448
    _flip_check(orc.NVFP4, q, k, v, c0, 48 * 6 / (2688 * l))
    # 448 E = 90: between 88 and 96, 2% from their midpoint 92; the code saturates (quotient 6.1)
    assert _run(orc.NVFP4, q, k, v, -math.log(90 / 448) / 18)[1] == 0.0


def test_mxfp4_code_tie():
    """MXFP4: the tile maximum's block has scale 2^-2, so key 1's quotient is 4 exp(-18 c) = 2.5 at
    exp(-18 c) = 0.625. Flip: P-hat 0.5 <-> 0.75, times 6, over l = 1.625."""
    q, k, v = _qkv(2, [6.0, 3.0], {(0, 0): 6.0, (1, 1): 6.0})
    c0 = -math.log(0.625) / 18
    _flip_check(orc.MXFP4, q, k, v, c0, 0.25 * 6 / 1.625)
    assert _run(orc.MXFP4, q, k, v, -math.log(0.7) / 18)[1] == 0.0  # quotient 2.8


def test_mxfp4_scale_boundary():
    """Key 4 (slot 32, block 1) alone in its block with E = 0.5, a power of two: the E8M0 scale is
    2^-3 (quotient 4, P-hat 0.5) or, just below, 2^-4 (quotient 8 saturates to 6, P-hat 0.375)."""
    kv = np.full(5, -384.0)
    kv[0], kv[4] = 6.0, 3.0
    q, k, v = _qkv(5, kv, {(0, 0): 6.0, (4, 1): 6.0})
    c0 = math.log(2) / 18
    _flip_check(orc.MXFP4, q, k, v, c0, 0.125 * 6 / 1.5)
    assert _run(orc.MXFP4, q, k, v, -math.log(0.45) / 18)[1] == 0.0  # E = 0.45: quotient 7.2 -> 6


def test_direct_p_bound_covers_the_normaliser():
    """Direct-P sums the rounded P, so a flip moves the normaliser too: the bound adds the head's
    largest |V-hat| to each key's. It must cover the flip; it is not tight."""
    q, k, v = _qkv(2, [6.0, 3.0], {(0, 0): 6.0, (1, 1): 6.0})
    c0 = -math.log(0.625) / 18
    # P-hat_1 in {0.5, 0.75}, l = 1 + P-hat_1: channel 1 moves 0.75*6/1.75 - 0.5*6/1.5 = 0.571;
    # the bound is |dP-hat| (|v| + max|V-hat|) / l with the side's own l, 1.5 or 1.75
    _flip_check(orc.MXFP4, q, k, v, c0, 0.75 * 6 / 1.75 - 0.5 * 6 / 1.5, direct_p=True,
                bound=(0.25 * 12 / 1.5, 0.25 * 12 / 1.75))
    assert _run(orc.MXFP4, q, k, v, -math.log(0.7) / 18, direct_p=True)[1] == 0.0


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4])
def test_window_grows_with_score_magnitude(fmt):
    """The same pair of keys 0.1% away from the code tie: no slack when the scores are of order 1,
    slack when a common term of 384 * 1536 * c (about 3e4) is added to both, since x - t is then
    resolved only to about 1e-2 in FP32."""
    e = 5 / 12 if fmt == orc.NVFP4 else 0.625
    c = -math.log(e * 1.001) / 18
    q, k, v = _qkv(2, [6.0, 3.0], {(0, 0): 6.0, (1, 1): 6.0})
    assert _run(fmt, q, k, v, c)[1] == 0.0
    q, k, v = _qkv(2, [6.0, 3.0], {(0, 0): 6.0, (1, 1): 6.0}, big=True)
    assert _run(fmt, q, k, v, c)[1] > 0.1
