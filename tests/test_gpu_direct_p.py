"""GPU parity of the Direct-P path (sage_fp4_quant x3 + sage_fp4_attn_fwd_direct_p, MXFP4) against
the oracle's Direct-P attention, to the same bar as the plain path: max-abs <= 2e-3 per output
element plus the oracle's per-row bound for probability roundings within 2^-14 of a boundary.
Also checks that the kernel's normaliser is really the rounded one: on inputs where the two
normalisers differ, the GPU output must follow the Direct-P oracle and not the plain one."""
import numpy as np
import pytest

import oracle as orc
from helpers import TOL, compare, gpu_attn, oracle_attn, sample_rows, say, workload

pytestmark = pytest.mark.gpu

MX = orc.MXFP4
SMALL = [((1, 2, 256, 64), 1), ((1, 2, 300, 128), 1), ((2, 3, 129, 64), 1), ((1, 1, 1, 128), 1),
         ((1, 2, 127, 64), 1), ((1, 1, 640, 128), 2)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,wl", SMALL)
def test_small_all_rows(causal, shape, wl):
    B, H, N, D = shape
    q, k, v = workload(wl, B=B, H=H, N=N, D=D)
    say(f"direct-p causal={causal} shape={shape}")
    g = gpu_attn(MX, q, k, v, causal, direct_p=True)
    assert np.all(np.isfinite(g))
    o, sl = oracle_attn(MX, q, k, v, causal, direct_p=True)
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"direct-p causal{causal} {shape}")


@pytest.mark.parametrize("wl,causal", [(2, False), (2, True), (3, False), (4, True)])
def test_full_size_sampled_rows(wl, causal):
    q, k, v = workload(wl)
    B, H, N, D = q.shape
    say(f"direct-p full workload {wl} causal={causal} shape={q.shape}")
    g = gpu_attn(MX, q, k, v, causal, direct_p=True)
    assert np.all(np.isfinite(g)), "unwritten or non-finite outputs"
    heads = [0, (B * H) // 2 + 1, B * H - 1]
    sub = workload(wl, heads=heads)
    rows_i = sample_rows(N, n_each=6, seed=wl)
    rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
    o, sl = oracle_attn(MX, *sub, causal, rows=rows, direct_p=True)
    gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
    compare(gr, o, sl, f"direct-p workload {wl} causal {causal}")


@pytest.mark.parametrize("N", [2048, 16384])
def test_long_sequences_sampled_rows(N):
    B, H, D = 1, 9, 128
    q, k, v = workload(2, B=B, H=H, N=N, D=D)
    say(f"direct-p sweep N={N}")
    for causal in (False, True):
        g = gpu_attn(MX, q, k, v, causal, direct_p=True)
        assert np.all(np.isfinite(g))
        heads = [0, 4, 8]
        rows_i = sample_rows(N, n_each=4, seed=N)
        rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
        sub = tuple(x[:, heads] for x in (q, k, v))
        o, sl = oracle_attn(MX, *sub, causal, rows=rows, direct_p=True)
        gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
        compare(gr, o, sl, f"direct-p N={N} causal {causal}")


def test_follows_the_rounded_normaliser():
    """Two keys per query. K's -2.88 quantises to -3 (E2M1 -6 x 2^-1), so the second key's score
    is -3/8 and its E = exp(-0.375) ~ 0.687; P-hat rounds that to 0.75 (E8M0 scale 1/4, code 3).
    With V rows +4 and -4 the output is 1/1.75 under Direct-P and 1/1.687 on the plain path."""
    B, H, N, D = 1, 4, 2, 64
    q = np.zeros((B, H, N, D), np.float16)
    k = np.zeros((B, H, N, D), np.float16)
    v = np.zeros((B, H, N, D), np.float16)
    q[..., 0] = 1.0
    k[:, :, 0, 0] = 0.0
    k[:, :, 1, 0] = -2.88
    v[:, :, 0, :] = 4.0
    v[:, :, 1, :] = -4.0
    g = gpu_attn(MX, q, k, v, False, direct_p=True)
    o_dp, sl = oracle_attn(MX, q, k, v, False, direct_p=True)
    o_plain, _ = oracle_attn(MX, q, k, v, False)
    compare(g.reshape(-1, D), o_dp.reshape(-1, D), sl, "two keys, Direct-P")
    gap = np.abs(o_dp - o_plain).max()
    say(f"  Direct-P vs plain oracle gap {gap:.4f}")
    np.testing.assert_allclose(o_dp[..., 0, :], 1 / 1.75, rtol=1e-6)
    assert gap > 10 * TOL
    assert np.abs(g.reshape(-1, D) - o_plain.reshape(-1, D)).max() > 5 * TOL


def test_q_zero_and_one_hot():
    _, k, v = workload(1, N=300, D=128)
    q = np.zeros_like(k)
    for causal in (False, True):
        g = gpu_attn(MX, q, k, v, causal, direct_p=True)
        o, sl = oracle_attn(MX, q, k, v, causal, direct_p=True)
        compare(g.reshape(-1, 128), o.reshape(-1, 128), sl, f"direct-p Q=0 causal {causal}")
    H, N, D = 128, 128, 64
    rng = np.random.default_rng(7)
    q = np.zeros((1, H, N, D), np.float16); q[0, :, :, 0] = 6.0
    k = np.zeros((1, H, N, D), np.float16); k[0, :, :, 0] = -48.0
    for h in range(H):
        k[0, h, h, 0] = 48.0
    v = (6.0 * rng.choice([-1.0, 1.0], size=(1, H, N, D))).astype(np.float16)
    g = gpu_attn(MX, q, k, v, False, direct_p=True)
    for h in range(H):
        np.testing.assert_allclose(g[0, h], np.broadcast_to(v[0, h, h].astype(np.float32), (N, D)), rtol=1e-6)


def test_f16_output_and_determinism():
    q, k, v = workload(1, N=300, D=128)
    a = gpu_attn(MX, q, k, v, True, direct_p=True)
    b = gpu_attn(MX, q, k, v, True, direct_p=True)
    assert np.array_equal(a, b)
    h = gpu_attn(MX, q, k, v, True, out_f32=False, direct_p=True)
    assert np.array_equal(h, a.astype(np.float16).astype(np.float32))
