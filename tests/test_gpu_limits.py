"""GPU parity at the limits the C ABI accepts: the longest sequence (N = 2^20, one head) and the
most heads (B*H = 65535, one token each), for every format, against the oracle on sampled rows.
These exercise the 32-bit per-head offsets and the largest grids the launchers build."""
import numpy as np
import pytest

import oracle as orc
from helpers import compare, gpu_attn, oracle_attn, say

pytestmark = pytest.mark.gpu

FMTS = [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True), (orc.MX4_PV8, False)]


def _normal(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float16)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
def test_longest_sequence(fmt, direct_p):
    N, D = 1 << 20, 64
    q, k, v = (_normal((1, 1, N, D), 900 + i) for i in range(3))
    for causal in (False, True):
        say(f"limits: N={N} fmt={fmt} direct_p={direct_p} causal={causal}")
        g = gpu_attn(fmt, q, k, v, causal, direct_p=direct_p)
        assert np.all(np.isfinite(g)), "unwritten or non-finite outputs"
        rows = np.array([0, 128, 654321, N - 1], np.int64)
        o, sl = oracle_attn(fmt, q, k, v, causal, rows=rows, direct_p=direct_p)
        compare(g.reshape(N, D)[rows], o, sl, f"N=2^20 fmt {fmt} dp {direct_p} causal {causal}")


@pytest.mark.parametrize("fmt,direct_p", FMTS)
def test_most_heads(fmt, direct_p):
    B, H, N, D = 1, 65535, 1, 128
    q, k, v = (_normal((B, H, N, D), 950 + i) for i in range(3))
    say(f"limits: B*H={B * H} fmt={fmt} direct_p={direct_p}")
    g = gpu_attn(fmt, q, k, v, False, direct_p=direct_p)
    o, sl = oracle_attn(fmt, q, k, v, False, direct_p=direct_p)
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"B*H=65535 fmt {fmt} dp {direct_p}")
