"""GPU parity of the FP4-QK / FP8-PV format (sage_fp4_quant x3 + sage_fp4_attn_fwd with
SAGE_FMT_MX4_PV8: MXFP4 Q and K, MXFP8 P and V) against the oracle's same format, to the bar of
the FP4 paths: max-abs <= 2e-3 per output element plus the oracle's per-row bound for
probability roundings within 2^-14 of a boundary. Small shapes on every row, the full-size
workloads and long sequences on sampled rows, degenerate inputs, and the accuracy ordering
against the unquantised reference (FP8 P and V beat FP4 P and V)."""
import numpy as np
import pytest

import oracle as orc
from helpers import compare, gpu_attn, oracle_attn, sample_rows, say, workload

pytestmark = pytest.mark.gpu

PV8 = orc.MX4_PV8
SMALL = [((1, 2, 256, 64), 1), ((1, 2, 300, 128), 1), ((2, 3, 129, 64), 1), ((1, 1, 1, 128), 1),
         ((1, 2, 127, 64), 1), ((1, 1, 640, 128), 2)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,wl", SMALL)
def test_small_all_rows(causal, shape, wl):
    B, H, N, D = shape
    q, k, v = workload(wl, B=B, H=H, N=N, D=D)
    say(f"pv8 causal={causal} shape={shape}")
    g = gpu_attn(PV8, q, k, v, causal)
    assert np.all(np.isfinite(g))
    o, sl = oracle_attn(PV8, q, k, v, causal)
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"pv8 causal{causal} {shape}")


@pytest.mark.parametrize("wl,causal", [(2, False), (2, True), (3, False), (4, True)])
def test_full_size_sampled_rows(wl, causal):
    q, k, v = workload(wl)
    B, H, N, D = q.shape
    say(f"pv8 full workload {wl} causal={causal} shape={q.shape}")
    g = gpu_attn(PV8, q, k, v, causal)
    assert np.all(np.isfinite(g)), "unwritten or non-finite outputs"
    heads = [0, (B * H) // 2 + 1, B * H - 1]
    sub = workload(wl, heads=heads)
    rows_i = sample_rows(N, n_each=6, seed=wl)
    rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
    o, sl = oracle_attn(PV8, *sub, causal, rows=rows)
    gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
    compare(gr, o, sl, f"pv8 workload {wl} causal {causal}")


@pytest.mark.parametrize("N", [2048, 16384])
def test_long_sequences_sampled_rows(N):
    B, H, D = 1, 9, 128
    q, k, v = workload(2, B=B, H=H, N=N, D=D)
    say(f"pv8 sweep N={N}")
    for causal in (False, True):
        g = gpu_attn(PV8, q, k, v, causal)
        assert np.all(np.isfinite(g))
        heads = [0, 4, 8]
        rows_i = sample_rows(N, n_each=4, seed=N)
        rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
        sub = tuple(x[:, heads] for x in (q, k, v))
        o, sl = oracle_attn(PV8, *sub, causal, rows=rows)
        gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
        compare(gr, o, sl, f"pv8 N={N} causal {causal}")


def test_q_zero_and_one_hot():
    _, k, v = workload(1, N=300, D=128)
    q = np.zeros_like(k)
    for causal in (False, True):
        g = gpu_attn(PV8, q, k, v, causal)
        o, sl = oracle_attn(PV8, q, k, v, causal)
        compare(g.reshape(-1, 128), o.reshape(-1, 128), sl, f"pv8 Q=0 causal {causal}")
    H, N, D = 128, 128, 64
    rng = np.random.default_rng(7)
    q = np.zeros((1, H, N, D), np.float16); q[0, :, :, 0] = 6.0
    k = np.zeros((1, H, N, D), np.float16); k[0, :, :, 0] = -48.0
    for h in range(H):
        k[0, h, h, 0] = 48.0
    v = (6.0 * rng.choice([-1.0, 1.0], size=(1, H, N, D))).astype(np.float16)
    g = gpu_attn(PV8, q, k, v, False)
    for h in range(H):
        np.testing.assert_allclose(g[0, h], np.broadcast_to(v[0, h, h].astype(np.float32), (N, D)), rtol=1e-6)


def test_f16_output_and_determinism():
    q, k, v = workload(1, N=300, D=128)
    a = gpu_attn(PV8, q, k, v, True)
    b = gpu_attn(PV8, q, k, v, True)
    assert np.array_equal(a, b)
    h = gpu_attn(PV8, q, k, v, True, out_f32=False)
    assert np.array_equal(h, a.astype(np.float16).astype(np.float32))


def test_fp8_pv_more_accurate_than_fp4_pv():
    q, k, v = workload(1)
    ref = orc.attn_ref_f64(q, k, v)

    def rel_l1(fmt):
        g = gpu_attn(fmt, q, k, v, False).astype(np.float64)
        return np.abs(g - ref).sum() / np.abs(ref).sum()

    e8, e4 = rel_l1(PV8), rel_l1(orc.MXFP4)
    say(f"  rel L1 vs FP64: FP8 PV {e8:.4f}, FP4 PV {e4:.4f}")
    assert e8 < 0.75 * e4
