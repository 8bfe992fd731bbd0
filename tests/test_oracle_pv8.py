"""Pins of the oracle's FP4-QK / FP8-PV variant (the rit.work page on FP4 FlashAttention-4,
section on what was done: in the page's distributed training, P and V stay in FP8 because every
variant with MXFP4 for them diverged). Reading: Q and K are MXFP4; P and V are MXFP8, i.e. E4M3
elements in 1x32 blocks with an E8M0 scale 2^(floor(log2 amax) - 8) (the OCP Microscaling rule).

Pins against things other than the oracle itself: torch's float8_e4m3fn cast (a library codec)
for the element rounding, numpy's log2 for the scale rule, an exhaustive nearest-value search
for the two-key closed form, exactly representable inputs, Q = 0 (uniform attention gives the
mean of V-hat, decoded with torch), one-hot attention, and the accuracy ordering against the
unquantised FP64 reference."""
import math

import numpy as np
import pytest
import torch

import oracle as orc

PV8 = orc.MX4_PV8
E4M3_VALUES = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def torch_e4m3_code(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def vhat_tokens_fp8(v_codes, v_scales, N):
    """V-hat in token order [B,H,N,D] float64, decoded with torch's float8 codecs."""
    v_codes, v_scales = orc.v_by_channel(v_codes, v_scales)
    B, H, D, Np = v_codes.shape
    vals = torch.from_numpy(v_codes).view(torch.float8_e4m3fn).double().numpy()
    sc = torch.from_numpy(v_scales).view(torch.float8_e8m0fnu).double().numpy()
    vd = vals * np.repeat(sc, 32, axis=-1)
    st = orc.slot_tokens()
    tok = np.array([(p // 128) * 128 + st[p % 128] for p in range(Np)])
    out = np.zeros((B, H, Np, D))
    out[:, :, tok, :] = np.transpose(vd, (0, 1, 3, 2))
    return out[:, :, :N, :]


def quant_all(q, k, v):
    return tuple(orc.quant(r, PV8, x) for r, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)))


def test_mx8_scale_rule_all_fp16_amax():
    f16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    pos = f16[np.isfinite(f16) & (f16 > 0)].astype(np.float64)
    want = np.floor(np.log2(pos)).astype(np.int64) - 8 + 127
    got = np.array([orc.lib().orc_mx8_scale(float(a)) for a in pos])
    assert np.array_equal(got, want)
    L = orc.lib()
    assert L.orc_mx8_scale(0.0) == 0 and L.orc_mx8_scale(1.0) == 119 and L.orc_mx8_scale(448.0) == 127
    assert L.orc_mx8_scale(2.0 ** -140) == 0 and L.orc_mx8_scale(3.0e38) == 127 + 127 - 8


def test_e4m3_element_rounding_against_torch():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * 4).astype(np.float16).astype(np.float32)
    L = orc.lib()
    for k in (-8, -3, 0, 2):
        s = 2.0 ** k
        got = np.array([L.orc_e4m3_quant(float(a), s) for a in x], np.uint8)
        y = np.abs(x) / np.float32(s)
        inr = y <= 448.0
        ref = torch_e4m3_code(y) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
        assert np.array_equal(got[inr], ref[inr])
        assert np.all((got[~inr] & 0x7F) == 0x7E)  # above 448: clamps to 448
    # every E4M3 midpoint (ties to the even code) and one FP32 ulp either side
    mids = ((E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2).astype(np.float32)
    ys = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    got = np.array([L.orc_e4m3_quant(float(a), 1.0) for a in ys], np.uint8)
    assert np.array_equal(got, torch_e4m3_code(ys))
    assert L.orc_e4m3_quant(-0.0, 1.0) == 0x80 and L.orc_e4m3_quant(0.0, 1.0) == 0
    assert L.orc_e4m3_quant(-1e-30, 1.0) == 0x80 and L.orc_e4m3_quant(3.0, 0.0) == 0


def test_block_quantiser_mx8():
    codes, s = orc.quant_block(PV8, np.array([1.0] + [0.25] * 31, np.float32))
    assert s == 119 and codes[0] == 0x78 and np.all(codes[1:] == 0x68)  # 256 and 64 in E4M3
    x = np.zeros(32, np.float32); x[3] = 1.9; x[7] = -0.1
    codes, s = orc.quant_block(PV8, x)
    assert s == 119 and codes[3] == 0x7E  # 1.9 * 256 = 486.4 clamps to 448
    assert codes[7] == (0x80 | int(torch_e4m3_code(np.float32(25.6))))
    codes, s = orc.quant_block(PV8, np.zeros(32, np.float32))
    assert s == 0 and np.all(codes == 0)


def test_q_and_k_are_mxfp4():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 2, 200, 64)).astype(np.float16)
    for role in (orc.ROLE_Q, orc.ROLE_K):
        a, b = orc.quant(role, PV8, x), orc.quant(role, orc.MXFP4, x)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_v_lossless_when_representable():
    """E4M3 numbers whose block maximum has a significand of at most 1.75 (so nothing clips at
    448) and which lie within the E4M3 range below it quantise exactly."""
    rng = np.random.default_rng(8)
    B, H, N, D = 1, 2, 300, 64
    v = rng.choice(np.array([0.5, -0.75, 1.0, 1.25, -2.0, 3.5, -4.0, 7.0], np.float16), size=(B, H, N, D))
    vc, vs = orc.quant(orc.ROLE_V, PV8, v)
    assert vc.shape == (B, H, 3, D, 128) and vs.shape == (B, H, 3, D, 4)
    vh = vhat_tokens_fp8(vc, vs, N)
    assert np.array_equal(vh, v.astype(np.float64))
    # token positions >= N (the padding of the last tile) are zero codes
    st = orc.slot_tokens()
    pad = [s for s in range(128) if 256 + st[s] >= N]
    assert np.all(vc[:, :, 2][..., pad] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_vhat(causal):
    """Q = 0: all scores 0, every visible E = 1, exactly 256 * 2^-8 in MXFP8: the output is the
    mean of V-hat over the visible keys."""
    rng = np.random.default_rng(21)
    B, H, N, D = 1, 2, 200, 128
    q = np.zeros((B, H, N, D), np.float16)
    k = rng.standard_normal((B, H, N, D)).astype(np.float16)
    v = rng.standard_normal((B, H, N, D)).astype(np.float16)
    Q, K, V = quant_all(q, k, v)
    vh = vhat_tokens_fp8(*V, N)
    got = orc.attn_fwd(PV8, Q, K, V, (B, H, N, D), causal=causal)
    if causal:
        want = np.cumsum(vh, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    else:
        want = np.broadcast_to(vh.mean(axis=2, keepdims=True), vh.shape)
    np.testing.assert_allclose(got, want, rtol=0, atol=2e-6)


def test_one_hot_rows():
    """Key h of head h scores 48 * 6 * c above the others: every other P value rounds to 0, so
    row outputs equal V-hat of key h exactly."""
    H, N, D = 4, 128, 64
    q = np.zeros((1, H, N, D), np.float16); q[0, :, :, 0] = 6.0
    k = np.zeros((1, H, N, D), np.float16); k[0, :, :, 0] = -48.0
    for h in range(H):
        k[0, h, 5 + 30 * h, 0] = 48.0
    rng = np.random.default_rng(2)
    v = rng.standard_normal((1, H, N, D)).astype(np.float16)
    Q, K, V = quant_all(q, k, v)
    vh = vhat_tokens_fp8(*V, N)
    got = orc.attn_fwd(PV8, Q, K, V, (1, H, N, D))
    for h in range(H):
        np.testing.assert_array_equal(got[0, h], np.broadcast_to(vh[0, h, 5 + 30 * h].astype(np.float32), (N, D)))


def e4m3_nearest(y):
    d = np.abs(E4M3_VALUES - y)
    i = int(np.argmin(d))
    assert np.sort(d)[1] > d[i], "tie"
    return E4M3_VALUES[i] if y <= 448.0 else 448.0


@pytest.mark.parametrize("k1", [3.0, 2.0, 1.0, 0.5, -2.0, -6.0])
def test_two_keys_closed_form(k1):
    """N = 2, D = 64, q = 4 e0, k0 = 4 e0, k1 = k1 e0 (E2M1 grid values: Q, K lossless). Scores
    x0 = 2, x1 = k1/2; the maximum has E = 1, so the block scale is 2^-8 and key 1's P is
    E1 = exp(x1 - 2) rounded to the E4M3 grid in units of 2^-8. The normaliser is 1 + E1."""
    N, D = 2, 64
    q = np.zeros((1, 1, N, D), np.float16); q[..., 0] = 4.0
    k = np.zeros((1, 1, N, D), np.float16); k[0, 0, 0, 0] = 4.0; k[0, 0, 1, 0] = k1
    v = np.random.default_rng(int(10 * k1) + 300).standard_normal((1, 1, N, D)).astype(np.float16)
    Q, K, V = quant_all(q, k, v)
    vh = vhat_tokens_fp8(*V, N)[0, 0]
    e1 = math.exp(k1 / 2.0 - 2.0)
    p1 = e4m3_nearest(e1 * 256.0) / 256.0
    want = (vh[0] + p1 * vh[1]) / (1.0 + e1)
    got = orc.attn_fwd(PV8, Q, K, V, (1, 1, N, D))[0, 0]
    for r in range(N):
        np.testing.assert_allclose(got[r], want, rtol=0, atol=2e-6)


def test_fp8_pv_is_more_accurate_than_fp4_pv():
    rng = np.random.default_rng(31)
    q, k, v = (rng.standard_normal((1, 2, 512, 64)).astype(np.float16) for _ in range(3))
    ref = orc.attn_ref_f64(q, k, v)

    def rel_l1(fmt):
        Q, K, V = (orc.quant(r, fmt, x) for r, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)))
        o = orc.attn_fwd(fmt, Q, K, V, q.shape).astype(np.float64)
        return np.abs(o - ref).sum() / np.abs(ref).sum()

    e8, e4 = rel_l1(PV8), rel_l1(orc.MXFP4)
    assert e8 < 0.75 * e4, (e8, e4)
