"""GPU parity on seeded random shapes (every row compared with the oracle at max-abs 2e-3, plus
half an fp16 ulp of the value for fp16 outputs): B in 1..3, H in 1..5, N in 1..700, D in {64, 128}, every format, Direct-P,
causal or not, fp32 or fp16 output. Catches indexing mistakes at unusual sizes (tails, one
token, odd head counts) that the fixed shape lists might miss."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_attention_amd import binding as bnd
from helpers import compare, oracle_attn, say, to_gpu

pytestmark = pytest.mark.gpu

FMTS = [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True), (orc.MX4_PV8, False)]


def case(i):
    r = np.random.default_rng(1000 + i)
    fmt, dp = FMTS[i % len(FMTS)]
    B, H = int(r.integers(1, 4)), int(r.integers(1, 6))
    edge = int(r.choice([1, 2, 63, 64, 65, 127, 128, 129, 255, 257]))
    N = edge if r.random() < 0.5 else int(r.integers(1, 701))
    D = int(r.choice([64, 128]))
    return fmt, dp, B, H, N, D, bool(r.integers(0, 2)), bool(r.integers(0, 2)), int(r.integers(0, 2**31))


@pytest.mark.parametrize("i", range(24))
def test_random_shape(i):
    fmt, dp, B, H, N, D, causal, f16_out, seed = case(i)
    say(f"random case {i}: fmt={fmt} dp={dp} B={B} H={H} N={N} D={D} causal={causal} f16={f16_out}")
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float16) for _ in range(3))
    Q, K, V = (bnd.quant(to_gpu(x), r, fmt) for x, r in ((q, 0), (k, 1), (v, 2)))
    out = torch.full((B, H, N, D), float("nan"), dtype=torch.float16 if f16_out else torch.float32,
                     device="cuda")
    bnd.attn_fwd_into(fmt, Q, K, V, (B, H, N, D), out, causal=causal, direct_p=dp)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g)), "unwritten outputs"
    o, sl = oracle_attn(fmt, q, k, v, causal, direct_p=dp)
    # the fp16 store rounds once more: half an fp16 ulp of each value
    extra = np.abs(o).reshape(-1, D).max(axis=1) * 2.0 ** -11 if f16_out else None
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"case {i}", extra=extra)
