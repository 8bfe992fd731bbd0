"""Pins of the oracle's row log-sum-exp (the normaliser of the online softmax, kept for a backward
pass and for merging partial results; DeepTech article, section on FP4 inference and its
hardware implementation, and the abstract's 8-bit training attention).

Pins: Q = 0 gives ln(number of visible keys) exactly; for the formats whose normaliser sums the
unquantised E, lse equals scipy's logsumexp of the scaled quantised scores (computed here from the
dequantised operands in float64); Direct-P's lse on two keys follows the closed form x0 + ln(1 + P1);
and two halves of the keys, computed as separate problems on whole 128-key tiles, merge with
their lse into the full result."""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as orc
from test_oracle_attention import vhat_tokens
from test_oracle_direct_p import e2m1_nearest

FMTS = [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True), (orc.MX4_PV8, False)]


def quant3(fmt, q, k, v):
    return tuple(orc.quant(r, fmt, x) for r, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)))


def qk_fmt(fmt):
    return orc.MXFP4 if fmt == orc.MX4_PV8 else fmt  # Q and K of the FP8-PV format are MXFP4


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_counts_visible_keys(fmt, direct_p, causal):
    N, D = 300, 64
    rng = np.random.default_rng(7)
    q = np.zeros((1, 2, N, D), np.float16)
    k = rng.standard_normal((1, 2, N, D)).astype(np.float16)
    v = rng.standard_normal((1, 2, N, D)).astype(np.float16)
    Q, K, V = quant3(fmt, q, k, v)
    _, lse = orc.attn_fwd(fmt, Q, K, V, (1, 2, N, D), causal=causal, direct_p=direct_p, want_lse=True)
    count = np.arange(1, N + 1) if causal else np.full(N, N)
    np.testing.assert_allclose(lse.reshape(2, N), np.log(np.broadcast_to(count, (2, N))), rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4, orc.MX4_PV8])
@pytest.mark.parametrize("causal", [False, True])
def test_plain_lse_is_logsumexp_of_scores(fmt, causal):
    """x = fl32(c * S) with S = Q-hat K-hat^T; the oracle forms S in FP32 from exact block
    partials, here it is formed in float64, hence the 1e-5 tolerance."""
    B, H, N, D = 1, 2, 333, 128
    rng = np.random.default_rng(11 + fmt)
    q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float16) for _ in range(3))
    Q, K, V = quant3(fmt, q, k, v)
    _, lse = orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), causal=causal, want_lse=True)
    qh = orc.dequant(qk_fmt(fmt), *Q)
    kh = orc.dequant(qk_fmt(fmt), *K)
    c = np.float32(1.0 / np.sqrt(D))
    x = (np.einsum("bhid,bhjd->bhij", qh, kh) * np.float64(c)).astype(np.float32).astype(np.float64)
    if causal:
        x = np.where(np.tril(np.ones((N, N), bool)), x, -np.inf)
    want = logsumexp(x, axis=-1).reshape(-1)
    np.testing.assert_allclose(lse, want, rtol=0, atol=1e-5)


@pytest.mark.parametrize("k1", [3.0, 1.0, -2.0])
def test_direct_p_two_keys(k1):
    """The two-key case of the Direct-P pins: scores x0 = 2 (the tile maximum, P0 = 1) and
    x1 = k1/2; the Direct-P normaliser is 1 + P1 with P1 the E2M1-rounded exp(x1 - 2) in units of
    1/4, the plain one 1 + exp(x1 - 2)."""
    N, D = 2, 64
    q = np.zeros((1, 1, N, D), np.float16); q[..., 0] = 4.0
    k = np.zeros((1, 1, N, D), np.float16); k[0, 0, 0, 0] = 4.0; k[0, 0, 1, 0] = k1
    v = np.random.default_rng(3).standard_normal((1, 1, N, D)).astype(np.float16)
    Q, K, V = quant3(orc.MXFP4, q, k, v)
    e1 = np.exp(k1 / 2.0 - 2.0)
    p1 = 0.25 * e2m1_nearest(e1 / 0.25)
    _, lse_dp = orc.attn_fwd(orc.MXFP4, Q, K, V, (1, 1, N, D), direct_p=True, want_lse=True)
    _, lse = orc.attn_fwd(orc.MXFP4, Q, K, V, (1, 1, N, D), want_lse=True)
    np.testing.assert_allclose(lse_dp, 2.0 + np.log1p(p1), rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, 2.0 + np.log1p(e1), rtol=0, atol=1e-6)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("n2", [128, 75])
def test_key_halves_merge(fmt, direct_p, n2):
    """Keys [0, 128) and [128, 128 + n2) as two separate problems over the first min(128, n2)
    query rows (quantisation is per row for Q and K and per 128-token tile for V, so the operands
    are the same codes), merged with their lse, equal the full problem's rows up to FP32 rounding."""
    D = 64
    N = 128 + n2
    rng = np.random.default_rng(100 + fmt + 10 * direct_p + n2)
    q, k, v = (rng.standard_normal((1, 2, N, D)).astype(np.float16) for _ in range(3))
    full = orc.attn_fwd(fmt, *quant3(fmt, q, k, v), (1, 2, N, D), direct_p=direct_p)
    rows = min(128, n2)
    qa = np.ascontiguousarray(q[:, :, :rows])
    parts = []
    for lo, n in ((0, 128), (128, n2)):
        kp = np.ascontiguousarray(k[:, :, lo:lo + n]); vp = np.ascontiguousarray(v[:, :, lo:lo + n])
        qp = np.zeros((1, 2, n, D), np.float16); qp[:, :, :rows] = qa
        o, l = orc.attn_fwd(fmt, *quant3(fmt, qp, kp, vp), (1, 2, n, D), direct_p=direct_p, want_lse=True)
        parts.append((o[:, :, :rows].astype(np.float64), l.reshape(2, n)[:, :rows]))
    (o1, l1), (o2, l2) = parts
    lse = np.logaddexp(l1, l2)
    merged = np.exp(l1 - lse)[None, :, :, None] * o1 + np.exp(l2 - lse)[None, :, :, None] * o2
    np.testing.assert_allclose(merged, full[:, :, :rows], rtol=0, atol=2e-6)
