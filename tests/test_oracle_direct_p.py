"""Pins of the oracle's Direct-P variant (the rit.work page on FP4 FlashAttention-4, section on
what was done: the scores go straight to the MXFP4 codes the second matmul consumes, and the
normaliser is computed from the same rounded values).

The P codes and block scales are those of the MXFP4 path; only the normaliser changes, from the
sum of the unquantised probabilities to the sum of the dequantised ones. Pins: a closed form for
two keys sharing one 32-slot block (the expected P value is rounded here by an independent
nearest-grid search), the mean of V when Q = 0 (every P value is exactly 1), and one-hot
attention (every P value but one rounds to 0)."""
import math

import numpy as np
import pytest

import oracle as orc
from test_oracle_attention import vhat_tokens

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1_nearest(y):
    """Nearest E2M1 magnitude to y >= 0 by exhaustive search (no tie occurs in these cases)."""
    d = [abs(y - g) for g in GRID]
    assert sorted(d)[0] < sorted(d)[1], "tie"
    return GRID[int(np.argmin(d))] if y <= 6.0 else 6.0


def quant_all(q, k, v):
    return tuple(orc.quant(r, orc.MXFP4, x) for r, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)))


@pytest.mark.parametrize("k1", [3.0, 2.0, 1.0, 0.5, -2.0])
def test_two_keys_closed_form(k1):
    """N = 2, D = 64: q = 4 e0, k0 = 4 e0, k1 = k1 e0 (all on the E2M1 grid, so Q and K quantise
    losslessly). Scores x0 = 2, x1 = k1/2 (c = 1/8); the tile maximum is key 0 with E = 1, which
    puts the block's E8M0 scale at 2^-2; key 1's value is E1 = exp(x1 - 2) rounded to the grid in
    units of 1/4. Direct-P divides by 1 + P1, the MXFP4 path by 1 + E1."""
    N, D = 2, 64
    q = np.zeros((1, 1, N, D), np.float16); q[..., 0] = 4.0
    k = np.zeros((1, 1, N, D), np.float16); k[0, 0, 0, 0] = 4.0; k[0, 0, 1, 0] = k1
    rng = np.random.default_rng(int(10 * k1) + 100)
    v = rng.standard_normal((1, 1, N, D)).astype(np.float16)
    Q, K, V = quant_all(q, k, v)
    vh = vhat_tokens(orc.MXFP4, *V, N)[0, 0]
    e1 = math.exp(k1 / 2.0 - 2.0)
    p1 = 0.25 * e2m1_nearest(e1 / 0.25)
    want_direct = (vh[0] + p1 * vh[1]) / (1.0 + p1)
    want_plain = (vh[0] + p1 * vh[1]) / (1.0 + e1)
    got_direct = orc.attn_fwd(orc.MXFP4, Q, K, V, (1, 1, N, D), direct_p=True)[0, 0]
    got_plain = orc.attn_fwd(orc.MXFP4, Q, K, V, (1, 1, N, D))[0, 0]
    for r in range(N):
        np.testing.assert_allclose(got_direct[r], want_direct, rtol=0, atol=2e-6)
        np.testing.assert_allclose(got_plain[r], want_plain, rtol=0, atol=2e-6)
    if p1 != e1:
        assert np.max(np.abs(got_direct - got_plain)) > 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_v(causal):
    """Q = 0: every score is 0, E = 1 for every visible key, which MXFP4 represents exactly
    (scale 2^-2, code 4), so the normaliser counts the visible keys and the output is the mean
    of the dequantised V rows (causal: prefix means), over several key tiles and a ragged tail."""
    N, D = 300, 128
    rng = np.random.default_rng(21)
    q = np.zeros((1, 2, N, D), np.float16)
    k = rng.standard_normal((1, 2, N, D)).astype(np.float16)
    v = rng.standard_normal((1, 2, N, D)).astype(np.float16)
    Q, K, V = quant_all(q, k, v)
    vh = vhat_tokens(orc.MXFP4, *V, N)
    got = orc.attn_fwd(orc.MXFP4, Q, K, V, (1, 2, N, D), causal=causal, direct_p=True)
    if causal:
        want = np.cumsum(vh, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    else:
        want = np.broadcast_to(vh.mean(axis=2, keepdims=True), vh.shape)
    np.testing.assert_allclose(got, want, rtol=0, atol=2e-6)


def test_one_hot_selects_one_row():
    """One key scores 30 above the others in every row: its P value is 1 and the rest round to
    0, so the output is that key's dequantised V row whether the normaliser sums rounded values
    or not."""
    N, D, H = 128, 64, 8
    q = np.zeros((1, H, N, D), np.float16); q[..., 0] = 6.0
    k = np.zeros((1, H, N, D), np.float16); k[..., 0] = -32.0
    for h in range(H):
        k[0, h, 17 * h % N, 0] = 32.0
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, H, N, D)).astype(np.float16)
    Q, K, V = quant_all(q, k, v)
    vh = vhat_tokens(orc.MXFP4, *V, N)
    got = orc.attn_fwd(orc.MXFP4, Q, K, V, (1, H, N, D), direct_p=True)
    for h in range(H):
        np.testing.assert_allclose(got[0, h], np.broadcast_to(vh[0, h, 17 * h % N], (N, D)), rtol=0, atol=1e-6)


def test_nvfp4_operands_rejected():
    with pytest.raises(ValueError):
        orc.attn_fwd(orc.NVFP4, None, None, None, (1, 1, 1, 64), direct_p=True)
