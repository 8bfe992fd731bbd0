"""Pins of the oracle's sm_scale argument (R10: x = fl32(c * S), c = fl32(1/sqrt(D)) unless given).

Doubling Q doubles every Q block scale exactly (NVFP4: E4M3(2 amax / 6) = 2 E4M3(amax / 6) below
the 448 clamp; MXFP4: the E8M0 exponent + 1) and leaves the codes alone, so S doubles exactly and
fl32(c * 2S) = fl32(2c * S): attention of 2Q at scale c is bit-identical to attention of Q at 2c.
An explicit c equal to the default gives the default result bit for bit."""
import numpy as np
import pytest

import oracle as orc

FMTS = [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True), (orc.MX4_PV8, False)]


def quant3(fmt, q, k, v):
    return tuple(orc.quant(r, fmt, x) for r, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)))


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_doubling_q_equals_doubling_scale(fmt, direct_p, causal):
    B, H, N, D = 1, 2, 200, 64
    rng = np.random.default_rng(5 + fmt + 3 * direct_p)
    q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float16) for _ in range(3))
    c = np.float32(0.11)
    a = orc.attn_fwd(fmt, *quant3(fmt, (q.astype(np.float32) * 2).astype(np.float16), k, v), (B, H, N, D),
                     causal=causal, sm_scale=float(c), direct_p=direct_p)
    b = orc.attn_fwd(fmt, *quant3(fmt, q, k, v), (B, H, N, D), causal=causal, sm_scale=float(2 * c),
                     direct_p=direct_p)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
def test_explicit_default_scale(fmt, direct_p):
    B, H, N, D = 1, 1, 130, 128
    rng = np.random.default_rng(77)
    q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float16) for _ in range(3))
    ops = quant3(fmt, q, k, v)
    a = orc.attn_fwd(fmt, *ops, (B, H, N, D), direct_p=direct_p)
    b = orc.attn_fwd(fmt, *ops, (B, H, N, D), sm_scale=float(np.float32(1.0 / np.sqrt(D))), direct_p=direct_p)
    assert np.array_equal(a, b)
