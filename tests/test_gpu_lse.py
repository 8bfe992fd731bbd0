"""GPU parity of sage_fp4_attn_fwd_lse: the row log-sum-exp against the oracle's, the output
against the plain entry point's (the same kernel, which only adds the store), and the merge of
two key halves computed as separate launches.

Bar for lse: |gpu - oracle| <= 1e-4 + 1e-6 |lse| (+ the oracle's lse slack with Direct-P, whose
normaliser sums rounded P values). Both sides sum l in FP32 in different orders (relative
differences of a few 1e-7 at these sizes) and the GPU forms (R + log2 l) ln 2 in FP32, whose
rounding at |lse| ~ 50 is a few 1e-6."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_attention_amd import binding as bnd
from helpers import sample_rows, say, to_gpu, workload

pytestmark = pytest.mark.gpu

FMTS = [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True), (orc.MX4_PV8, False)]


def gpu_lse(fmt, q, k, v, causal, direct_p, out_dtype=torch.float32):
    B, H, N, D = q.shape
    Q, K, V = (bnd.quant(to_gpu(x), r, fmt) for x, r in ((q, 0), (k, 1), (v, 2)))
    out = torch.full((B, H, N, D), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B * H * N,), float("nan"), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(fmt, Q, K, V, (B, H, N, D), out, causal=causal, direct_p=direct_p, lse=lse)
    ref = torch.full_like(out, float("nan"))
    bnd.attn_fwd_into(fmt, Q, K, V, (B, H, N, D), ref, causal=causal, direct_p=direct_p)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "the lse entry point changed the output"
    return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)


def oracle_lse(fmt, q, k, v, causal, direct_p, rows=None):
    B, H, N, D = q.shape
    Q, K, V = (orc.quant(r, fmt, x) for x, r in ((q, 0), (k, 1), (v, 2)))
    _, _, lse, lsl = orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), causal=causal, rows=rows, want_slack=True,
                                  direct_p=direct_p, want_lse=True)
    return lse, lsl


def check(g, o, slack, what):
    err = np.abs(g - o)
    bound = 1e-4 + 1e-6 * np.abs(o) + slack
    say(f"  [{what}] max |lse err| {err.max():.3g} over {err.size} rows")
    assert np.all(np.isfinite(g)), "unwritten lse rows"
    assert np.all(err <= bound), f"{what}: worst row {np.argmax(err - bound)} err {err.max()}"


@pytest.mark.parametrize("fmt,direct_p", FMTS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (2, 3, 129, 64), (1, 2, 300, 128), (1, 1, 1, 128)])
def test_small_all_rows(fmt, direct_p, causal, shape):
    B, H, N, D = shape
    q, k, v = workload(1, B=B, H=H, N=N, D=D)
    say(f"lse fmt={fmt} direct_p={direct_p} causal={causal} shape={shape}")
    _, g = gpu_lse(fmt, q, k, v, causal, direct_p)
    o, sl = oracle_lse(fmt, q, k, v, causal, direct_p)
    check(g, o, sl, f"fmt{fmt} dp{direct_p} causal{causal} {shape}")


@pytest.mark.parametrize("fmt,direct_p", FMTS)
def test_key_halves_merge(fmt, direct_p):
    """Keys [0, 128) and [128, 256) as two launches over the first 128 query rows, merged with
    their lse, against the launch over all 256 keys (all on the GPU)."""
    D = 128
    rng = np.random.default_rng(40 + fmt + 5 * direct_p)
    q, k, v = (rng.standard_normal((1, 4, 256, D)).astype(np.float16) for _ in range(3))
    full, _ = gpu_lse(fmt, q, k, v, False, direct_p)
    parts = []
    for lo in (0, 128):
        sl = slice(lo, lo + 128)
        o, l = gpu_lse(fmt, np.ascontiguousarray(q[:, :, :128]), np.ascontiguousarray(k[:, :, sl]),
                       np.ascontiguousarray(v[:, :, sl]), False, direct_p)
        parts.append((o.astype(np.float64), l.reshape(4, 128)))
    (o1, l1), (o2, l2) = parts
    lse = np.logaddexp(l1, l2)
    merged = np.exp(l1 - lse)[None, :, :, None] * o1 + np.exp(l2 - lse)[None, :, :, None] * o2
    err = np.abs(merged - full[:, :, :128]).max()
    say(f"  [merge fmt{fmt} dp{direct_p}] max err {err:.3g}")
    assert err <= 2e-5


@pytest.mark.parametrize("wl,fmt,direct_p,causal", [(2, orc.NVFP4, False, False), (4, orc.NVFP4, False, True),
                                                    (2, orc.MXFP4, True, True), (3, orc.MX4_PV8, False, False)])
def test_full_size_sampled_rows(wl, fmt, direct_p, causal):
    q, k, v = workload(wl)
    B, H, N, D = q.shape
    say(f"lse full workload {wl} fmt={fmt} direct_p={direct_p} causal={causal}")
    _, g = gpu_lse(fmt, q, k, v, causal, direct_p, out_dtype=torch.float16)
    heads = [0, (B * H) // 2 + 1, B * H - 1]
    sub = workload(wl, heads=heads)
    rows_i = sample_rows(N, n_each=6, seed=wl)
    rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
    o, sl = oracle_lse(fmt, *sub, causal, direct_p, rows=rows)
    gr = np.concatenate([g.reshape(B * H, N)[h][rows_i] for h in heads])
    check(gr, o, sl, f"workload {wl} fmt {fmt} dp {direct_p} causal {causal}")
