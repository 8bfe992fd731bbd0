"""GPU parity of the full hot path (sage_fp4_quant x3 + sage_fp4_attn_fwd) against the oracle.

Bar: max-abs <= 2e-3 on every compared row. Small shapes are compared on every row; the full-size
workloads, in the configuration bench.py times, on sampled rows the oracle computes one by one.
The oracle's slack (its bound on P decisions within FP32 resolution of a boundary) is reported,
not added: on these inputs no such decision moves a row by more than a few 1e-4."""
import numpy as np
import pytest

import oracle as orc
from helpers import compare, gpu_attn, oracle_attn, sample_rows, say, workload

pytestmark = pytest.mark.gpu

SMALL = [((1, 2, 256, 64), 1), ((1, 2, 300, 128), 1), ((2, 3, 129, 64), 1), ((1, 1, 1, 128), 1),
         ((1, 2, 127, 64), 1), ((1, 1, 640, 128), 2)]


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,wl", SMALL)
def test_small_all_rows(fmt, causal, shape, wl):
    B, H, N, D = shape
    q, k, v = workload(wl, B=B, H=H, N=N, D=D)
    say(f"attn fmt={fmt} causal={causal} shape={shape}")
    g = gpu_attn(fmt, q, k, v, causal)
    assert np.all(np.isfinite(g))
    o, sl = oracle_attn(fmt, q, k, v, causal)
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"fmt{fmt} causal{causal} {shape}")


@pytest.mark.parametrize("wl,fmt,causal", [(1, orc.NVFP4, False), (5, orc.MXFP4, False)])
def test_workloads_1_and_5_all_rows(wl, fmt, causal):
    q, k, v = workload(wl)
    B, H, N, D = q.shape
    say(f"attn workload {wl}")
    g = gpu_attn(fmt, q, k, v, causal)
    o, sl = oracle_attn(fmt, q, k, v, causal)
    compare(g.reshape(-1, D), o.reshape(-1, D), sl, f"workload {wl}")


FULL = [(2, orc.NVFP4, False), (2, orc.NVFP4, True), (3, orc.NVFP4, False), (4, orc.NVFP4, True),
        (2, orc.MXFP4, False), (2, orc.MXFP4, True), (3, orc.MXFP4, False), (4, orc.MXFP4, True)]


@pytest.mark.parametrize("wl,fmt,causal", FULL)
def test_full_size_sampled_rows(wl, fmt, causal):
    q, k, v = workload(wl)
    B, H, N, D = q.shape
    say(f"attn full workload {wl} fmt={fmt} causal={causal} shape={q.shape}")
    g = gpu_attn(fmt, q, k, v, causal)
    assert np.all(np.isfinite(g)), "unwritten or non-finite outputs"
    heads = [0, (B * H) // 2 + 1, B * H - 1]
    sub = workload(wl, heads=heads)
    rows_i = sample_rows(N, n_each=6, seed=wl)
    rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
    o, sl = oracle_attn(fmt, *sub, causal, rows=rows)
    gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
    compare(gr, o, sl, f"workload {wl} fmt {fmt} causal {causal}")


@pytest.mark.parametrize("N", [1024, 2048, 8192, 16384])
@pytest.mark.parametrize("causal", [False, True])
def test_sweep_lengths_sampled_rows(N, causal):
    """The sequence lengths of the kernel sweep (D = 128, N(0,1) data) with 9 heads, an odd head
    count, so the workgroup count is not a multiple of the 8 XCDs."""
    B, H, D = 1, 9, 128
    q, k, v = workload(2, B=B, H=H, N=N, D=D)
    say(f"attn sweep N={N} causal={causal}")
    for fmt in (orc.NVFP4, orc.MXFP4):
        g = gpu_attn(fmt, q, k, v, causal)
        assert np.all(np.isfinite(g)), "unwritten or non-finite outputs"
        heads = [0, 4, 8]
        rows_i = sample_rows(N, n_each=4, seed=N)
        rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
        sub = tuple(x[:, heads] for x in (q, k, v))
        o, sl = oracle_attn(fmt, *sub, causal, rows=rows)
        gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
        compare(gr, o, sl, f"sweep N={N} fmt {fmt} causal {causal}")


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4])
def test_q_zero_and_one_hot(fmt):
    """Degenerate inputs: Q = 0 (all scores equal) and one-hot attention at every slot."""
    _, k, v = workload(1, N=300, D=128)
    q = np.zeros_like(k)
    for causal in (False, True):
        g = gpu_attn(fmt, q, k, v, causal)
        o, sl = oracle_attn(fmt, q, k, v, causal)
        compare(g.reshape(-1, 128), o.reshape(-1, 128), sl, f"Q=0 causal {causal}")
    H, N, D = 128, 128, 64
    rng = np.random.default_rng(7)
    q = np.zeros((1, H, N, D), np.float16); q[0, :, :, 0] = 6.0
    k = np.zeros((1, H, N, D), np.float16); k[0, :, :, 0] = -48.0
    for h in range(H):
        k[0, h, h, 0] = 48.0
    v = (6.0 * rng.choice([-1.0, 1.0], size=(1, H, N, D))).astype(np.float16)
    g = gpu_attn(fmt, q, k, v, False)
    for h in range(H):
        np.testing.assert_allclose(g[0, h], np.broadcast_to(v[0, h, h].astype(np.float32), (N, D)), rtol=1e-6)


def test_determinism_and_f16_output():
    q, k, v = workload(1, N=300, D=128)
    a = gpu_attn(orc.NVFP4, q, k, v, True)
    b = gpu_attn(orc.NVFP4, q, k, v, True)
    assert np.array_equal(a, b)
    h = gpu_attn(orc.NVFP4, q, k, v, True, out_f32=False)
    assert np.array_equal(h, a.astype(np.float16).astype(np.float32))


def _metrics(a, b):
    a = a.reshape(-1).astype(np.float64); b = b.reshape(-1).astype(np.float64)
    return float(a @ b / np.sqrt((a @ a) * (b @ b))), float(np.abs(a - b).sum() / np.abs(b).sum())


def test_accuracy_nvfp4_vs_mxfp4_against_full_precision():
    """The pages' direction (NVFP4 more accurate than MXFP4) on the GPU path, workloads 1 and 3."""
    q, k, v = workload(1)
    ref = orc.attn_ref_f64(q, k, v)
    cn, ln = _metrics(gpu_attn(orc.NVFP4, q, k, v, False), ref)
    cm, lm = _metrics(gpu_attn(orc.MXFP4, q, k, v, False), ref)
    say(f"  workload 1: NVFP4 cos {cn:.5f} relL1 {ln:.4f} | MXFP4 cos {cm:.5f} relL1 {lm:.4f}")
    assert cn > cm and ln < lm and cn > 0.975
    q, k, v = workload(3)
    B, H, N, D = q.shape
    heads = [0, 17, 47]
    sub = workload(3, heads=heads)
    rows_i = sample_rows(N, n_each=16, seed=3)
    rows = np.concatenate([u * N + rows_i for u in range(len(heads))])
    ref = orc.attn_ref_f64(*sub, rows=rows)
    res = {}
    for fmt in (orc.NVFP4, orc.MXFP4):
        g = gpu_attn(fmt, q, k, v, False)
        gr = np.concatenate([g.reshape(B * H, N, D)[h][rows_i] for h in heads])
        res[fmt] = _metrics(gr, ref)
    say(f"  workload 3 (sampled rows): NVFP4 {res[0]} | MXFP4 {res[1]}")
    assert res[0][0] > res[1][0]


@pytest.mark.parametrize("fmt,direct_p", [(orc.NVFP4, False), (orc.MXFP4, False), (orc.MXFP4, True),
                                          (orc.MX4_PV8, False)])
@pytest.mark.parametrize("causal", [False, True])
def test_bench_configuration_f16_output(fmt, direct_p, causal):
    """bench.py times the fp16-output instances at B4 H32 N4096 D128. Their output must be the
    fp32-output instance's (checked against the oracle above and in the Direct-P / FP8-PV files)
    rounded to fp16, bit for bit, on every element."""
    q, k, v = workload(2)
    say(f"bench configuration fmt={fmt} direct_p={direct_p} causal={causal}")
    a = gpu_attn(fmt, q, k, v, causal, direct_p=direct_p)
    h = gpu_attn(fmt, q, k, v, causal, out_f32=False, direct_p=direct_p)
    assert np.array_equal(h, a.astype(np.float16).astype(np.float32))
