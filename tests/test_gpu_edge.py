"""GPU parity on edge cases of the attention entry points, against the oracle:
  - explicit sm_scale values (the boundary's sm_scale argument; sm_scale <= 0 selects 1/sqrt(D));
  - score gaps so large that whole key tiles fall more than 2^64 below the running maximum (the
    kernels drop them) and whole P blocks underflow;
  - inputs large enough to saturate the E4M3 scales, and inputs so small that the block scales
    underflow to zero;
  - scores of order 1e5.
Bar: max-abs 2e-3 plus the oracle's per-row slack. These inputs make attention sharp (a row's
weight sits on a few keys, so one P code moves the output by far more than 2e-3) or make the
scores large (FP32 resolves x - t only to about 2^-20 (|x| + |t|)), so a P decision that lies
within that resolution of its boundary may go either way in a correct implementation; the slack
is the oracle's bound on the effect of each such decision (pinned in test_oracle_slack.py)."""
import numpy as np
import pytest

import oracle as orc
from helpers import compare, gpu_attn, oracle_attn, say

pytestmark = pytest.mark.gpu

FMTS = [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True), (orc.MX4_PV8, False)]


def gpu_attn_scaled(fmt, q, k, v, causal, sm_scale, direct_p):
    import torch
    from bit_attention_amd import binding as bnd
    from helpers import to_gpu
    B, H, N, D = q.shape
    Q, K, V = (bnd.quant(to_gpu(x), r, fmt) for x, r in ((q, 0), (k, 1), (v, 2)))
    out = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(fmt, Q, K, V, (B, H, N, D), out, causal=causal, sm_scale=sm_scale, direct_p=direct_p)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_scaled(fmt, q, k, v, causal, sm_scale, direct_p):
    B, H, N, D = q.shape
    Q, K, V = (orc.quant(r, fmt, x) for x, r in ((q, 0), (k, 1), (v, 2)))
    return orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), causal=causal, sm_scale=sm_scale, want_slack=True,
                        direct_p=direct_p)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("sm_scale", [0.05, 0.3, 1.0])
@pytest.mark.parametrize("causal", [False, True])
def test_explicit_sm_scale(fmt, direct_p, sm_scale, causal):
    rng = np.random.default_rng(int(sm_scale * 100) + fmt)
    q, k, v = (rng.standard_normal((1, 2, 300, 64)).astype(np.float16) for _ in range(3))
    say(f"sm_scale {sm_scale} fmt={fmt} dp={direct_p} causal={causal}")
    g = gpu_attn_scaled(fmt, q, k, v, causal, sm_scale, direct_p)
    o, sl = oracle_scaled(fmt, q, k, v, causal, sm_scale, direct_p)
    compare(g.reshape(-1, 64), o.reshape(-1, 64), sl, f"sm_scale {sm_scale} fmt{fmt} dp{direct_p} c{causal}",
            use_slack=True)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("causal", [False, True])
def test_rejected_tiles_and_underflowing_blocks(fmt, direct_p, causal):
    """Key 5 scores 512 (natural units) above the rest of tile 0 and 1024 above tile 1, so tile 1
    lies far more than 2^64 below the maximum and every P block without key 5 underflows; rows
    that cannot see key 5 (causal) attend uniformly to tile 0's other keys."""
    N, D = 256, 64
    q = np.zeros((1, 2, N, D), np.float16); q[..., 0] = 64.0
    k = np.zeros((1, 2, N, D), np.float16); k[0, :, 5, 0] = 64.0; k[0, :, 128:, 0] = -64.0
    v = np.random.default_rng(9).standard_normal((1, 2, N, D)).astype(np.float16)
    g = gpu_attn(fmt, q, k, v, causal, direct_p=direct_p)
    assert np.all(np.isfinite(g))
    o, sl = oracle_attn(fmt, q, k, v, causal, direct_p=direct_p)
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"rejected tiles fmt{fmt} dp{direct_p} c{causal}",
            use_slack=True)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("case", ["q_saturated", "k_saturated", "subnormal"])
def test_extreme_input_magnitudes(fmt, direct_p, case):
    """Q (or K) at 300 * N(0,1) saturates NVFP4's E4M3 scales (amax / 6 > 448) while the other
    operand at 0.01 * N(0,1) keeps the scaled scores moderate; Q, K and V at 1e-5 * N(0,1) lie in
    fp16's subnormal range, where the NVFP4 block scales round to zero (every code 0, so all
    scores are 0 and V-hat is 0) and MXFP4 keeps tiny E8M0 scales."""
    rng = np.random.default_rng(31 + fmt)
    shape = (1, 2, 200, 128)
    big, small = rng.standard_normal(shape) * 300.0, rng.standard_normal(shape) * 0.01
    if case == "q_saturated":
        q, k, v = big, small, rng.standard_normal(shape)
    elif case == "k_saturated":
        q, k, v = small, big, rng.standard_normal(shape)
    else:
        q, k, v = (rng.standard_normal(shape) * 1e-5 for _ in range(3))
    q, k, v = (x.astype(np.float16) for x in (q, k, v))
    g = gpu_attn(fmt, q, k, v, False, direct_p=direct_p)
    assert np.all(np.isfinite(g))
    o, sl = oracle_attn(fmt, q, k, v, False, direct_p=direct_p)
    compare(g.reshape(-1, 128), o.reshape(-1, 128), sl, f"{case} fmt{fmt} dp{direct_p}", use_slack=True)


@pytest.mark.parametrize("fmt,direct_p", FMTS)
def test_huge_scores(fmt, direct_p):
    """Q and K both at 300 * N(0,1): scaled scores reach ~1e5. Rows are nearly one-hot, and the
    tile maximum must still get E = 1 exactly (it sets the normaliser); the other decisions carry
    the oracle's magnitude-scaled slack."""
    rng = np.random.default_rng(61 + fmt)
    shape = (1, 2, 200, 128)
    q, k = ((rng.standard_normal(shape) * 300.0).astype(np.float16) for _ in range(2))
    v = rng.standard_normal(shape).astype(np.float16)
    g = gpu_attn(fmt, q, k, v, False, direct_p=direct_p)
    assert np.all(np.isfinite(g))
    o, sl = oracle_attn(fmt, q, k, v, False, direct_p=direct_p)
    compare(g.reshape(-1, 128), o.reshape(-1, 128), sl, f"huge scores fmt{fmt} dp{direct_p}", use_slack=True)
