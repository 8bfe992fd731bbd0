"""GPU parity of sage_fp4_quant: codes and scales bit-exact against the oracle.

Covers every positive and negative fp16 value against every E4M3 scale (NVFP4) and against every
power-of-two scale fp16 inputs can produce (MXFP4), MXFP8 V blocks over the whole fp16 range
(clipping blocks included), the saturation and underflow regions, zeros and signed zeros, every
workload's tensors (whole small ones; sampled heads of the full-size ones, which the quantiser
treats independently), ragged token counts and both head sizes."""
import numpy as np
import pytest

import oracle as orc
from helpers import gpu_quant, say, workload

pytestmark = pytest.mark.gpu

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
PV8 = orc.MX4_PV8
FIN = ALL[np.isfinite(ALL)]


def _blocks_for_scale_nv(rng):
    """Rows of 64 channels (4 NVFP4 blocks). For each E4M3 scale s: blocks holding 6s (so the
    scale is exactly s) and every fp16 value of magnitude <= 6s, both signs."""
    vals = []
    e4m3 = np.array([orc.lib().orc_e4m3_decode(b) for b in range(1, 127)], np.float64)
    for s in e4m3:
        amax = np.float16(6 * s)
        xs = FIN[np.abs(FIN.astype(np.float64)) <= float(amax)]
        xs = xs[rng.permutation(len(xs))]
        nb = (len(xs) + 14) // 15
        pad = np.zeros(nb * 15, np.float16)
        pad[:len(xs)] = xs
        blocks = pad.reshape(nb, 15)
        pos = rng.integers(0, 16, nb)
        full = np.zeros((nb, 16), np.float16)
        for i in range(nb):
            full[i] = np.insert(blocks[i], pos[i], amax * (1 if rng.random() < 0.5 else -1))
        vals.append(full)
    # saturated scales (amax > 2688), underflowing scales (amax/6 < 2^-10), zeros, signed zeros
    big = (rng.uniform(2689, 65504, (512, 16)) * rng.choice([-1, 1], (512, 16))).astype(np.float16)
    tiny = (rng.uniform(0, 6 * 2.0 ** -10, (512, 16)) * rng.choice([-1, 1], (512, 16))).astype(np.float16)
    zeros = np.zeros((64, 16), np.float16)
    zeros[::2] = np.float16(-0.0)
    edge = np.array([[65504, -65504] + [0] * 14, [6 * 2.0 ** -10] + [0] * 15], np.float16)
    vals += [big, tiny, zeros, edge]
    allb = np.concatenate(vals)
    nrow = (len(allb) + 3) // 4
    out = np.zeros((nrow * 4, 16), np.float16)
    out[:len(allb)] = allb
    return out.reshape(1, 1, nrow, 64)


def test_nvfp4_every_fp16_against_every_e4m3_scale():
    x = _blocks_for_scale_nv(np.random.default_rng(11))
    say(f"nvfp4 exhaustive table: {x.shape}")
    gc, gs = gpu_quant(x, orc.ROLE_Q, orc.NVFP4)
    oc, os_ = orc.quant(orc.ROLE_Q, orc.NVFP4, x)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def test_mxfp4_every_fp16_against_every_scale():
    rng = np.random.default_rng(12)
    vals = []
    for E in range(-24, 16):  # floor(log2 amax) over the fp16 range
        lo, hi = 2.0 ** E, min(2.0 ** (E + 1), 65504.0 + 1)
        amaxs = FIN[(np.abs(FIN.astype(np.float64)) >= lo) & (np.abs(FIN.astype(np.float64)) < hi)]
        amax = amaxs[np.argmax(np.abs(amaxs.astype(np.float64)))]
        xs = FIN[np.abs(FIN.astype(np.float64)) <= abs(float(amax))]
        xs = xs[rng.permutation(len(xs))][: 31 * 400]
        nb = (len(xs) + 30) // 31
        pad = np.zeros(nb * 31, np.float16)
        pad[:len(xs)] = xs
        blk = np.concatenate([pad.reshape(nb, 31), np.full((nb, 1), amax, np.float16)], axis=1)
        vals.append(blk)
    allb = np.concatenate(vals)
    nrow = (len(allb) + 1) // 2
    out = np.zeros((nrow * 2, 32), np.float16)
    out[:len(allb)] = allb
    x = out.reshape(1, 1, nrow, 64)
    say(f"mxfp4 exhaustive table: {x.shape}")
    gc, gs = gpu_quant(x, orc.ROLE_K, orc.MXFP4)
    oc, os_ = orc.quant(orc.ROLE_K, orc.MXFP4, x)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def test_mxfp8_v_blocks_over_the_fp16_range():
    """V of the FP8-PV format: per (channel, 32-slot block) a random binade for the block maximum
    (all of fp16's), its significand drawn from {1, 1.75, 1.8125, 1.999} and random ones (so some
    blocks clip at 448), the other values spread over 24 binades below it, both signs, zeros
    and signed zeros; written to token order through the slot order."""
    rng = np.random.default_rng(13)
    D, ntile = 64, 48
    nb = ntile * 4
    E = rng.integers(-24, 16, (D, nb))
    sig = rng.choice([1.0, 1.75, 1.8125, 1.999, 1.5, 1.25], (D, nb))
    vals = np.empty((D, nb, 32), np.float64)
    for d in range(D):
        for b in range(nb):
            k = rng.integers(0, 24, 32)
            m = rng.uniform(1, 2, 32)
            v = m * 2.0 ** (E[d, b] - k) * rng.choice([-1.0, 1.0], 32)
            v[rng.integers(0, 32)] = sig[d, b] * 2.0 ** E[d, b] * rng.choice([-1.0, 1.0])
            v[rng.random(32) < 0.03] = 0.0
            vals[d, b] = v
    vals = np.clip(vals, -65504, 65504).astype(np.float16)
    vals[vals == 0] = np.where(rng.random((vals == 0).sum()) < 0.5, np.float16(-0.0), np.float16(0.0))
    st = orc.slot_tokens()
    x = np.zeros((1, 1, ntile * 128, D), np.float16)
    for t in range(ntile):
        blk = vals[:, 4 * t:4 * t + 4, :].reshape(D, 128)  # [d, slot]
        x[0, 0, t * 128 + st, :] = blk.T
    say(f"mxfp8 V table: {x.shape}")
    gc, gs = gpu_quant(x, orc.ROLE_V, PV8)
    oc, os_ = orc.quant(orc.ROLE_V, PV8, x)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4, PV8])
@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (2, 3, 300, 128), (1, 1, 1, 64), (1, 2, 129, 128)])
def test_small_shapes_all_roles(fmt, shape):
    B, H, N, D = shape
    q, k, v = workload(1, B=B, H=H, N=N, D=D)
    for role, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)):
        say(f"quant fmt={fmt} role={role} shape={shape}")
        gc, gs = gpu_quant(x, role, fmt)
        oc, os_ = orc.quant(role, fmt, x)
        assert np.array_equal(gs, os_), (role, shape)
        assert np.array_equal(gc, oc), (role, shape)


@pytest.mark.parametrize("wl,fmt", [(2, orc.NVFP4), (3, orc.NVFP4), (4, orc.NVFP4), (3, orc.MXFP4), (4, PV8)])
def test_full_size_workloads_sampled_heads(wl, fmt):
    """Full-size tensors through the GPU quantiser; the oracle checks a few whole heads."""
    q, k, v = workload(wl)
    B, H, N, D = q.shape
    heads = [0, (B * H) // 2, B * H - 1]
    sub = workload(wl, heads=heads)
    for role, x, xs in ((orc.ROLE_Q, q, sub[0]), (orc.ROLE_K, k, sub[1]), (orc.ROLE_V, v, sub[2])):
        say(f"quant workload {wl} fmt={fmt} role={role} shape={x.shape}")
        gc, gs = gpu_quant(x, role, fmt)
        oc, os_ = orc.quant(role, fmt, xs)
        gcf = gc.reshape(B * H, *gc.shape[2:])[heads]
        gsf = gs.reshape(B * H, *gs.shape[2:])[heads]
        assert np.array_equal(gsf, os_[0]), (wl, role)
        assert np.array_equal(gcf, oc[0]), (wl, role)


def test_quant_is_deterministic():
    q, k, v = workload(1, N=300, D=128)
    for role, x in ((orc.ROLE_Q, q), (orc.ROLE_V, v)):
        a = gpu_quant(x, role, orc.NVFP4)
        b = gpu_quant(x, role, orc.NVFP4)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
