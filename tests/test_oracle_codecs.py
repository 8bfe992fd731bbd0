"""Pins of the oracle's element codecs and block quantisers against things other than itself:
the torch float8 codecs (library routines), the OCP tables, closed-form tie cases and an
independent piecewise round-half-even formulation of E2M1 rounding.

Formats: SageAttention3, DeepTech article, section on FP4 data types (NVFP4 = E2M1 values,
1x16 blocks, E4M3 scales; MXFP4 = E2M1, 1x32, E8M0) and section on the two FP4 obstacles
(FP4 represents only 15 distinct values)."""
import numpy as np
import pytest
import torch

import oracle as orc

ALL_F16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
POS_F16 = ALL_F16[np.isfinite(ALL_F16) & (ALL_F16 > 0)]


def test_e2m1_has_fifteen_values():
    vals = [orc.lib().orc_e2m1_decode(c) for c in range(16)]
    assert len(set(vals)) == 15  # +0 and -0 compare equal
    # OCP Microscaling v1.0, E2M1 table (magnitudes), sign in bit 3
    assert vals[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert vals[8:] == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e4m3_decode_matches_torch():
    got = np.array([orc.lib().orc_e4m3_decode(b) for b in range(256)], np.float32)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(got, ref, equal_nan=True)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e8m0_decode_matches_torch():
    got = np.array([orc.lib().orc_e8m0_decode(b) for b in range(256)], np.float32)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    assert np.array_equal(got[:255], ref[:255])
    assert np.isnan(got[255])


def _torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_scale_rule_all_fp16_amax():
    """NVFP4 scale of every positive fp16 amax: fl32(amax/6) rounded to E4M3 (RNE), clamped."""
    y = (POS_F16.astype(np.float32) / np.float32(6.0)).astype(np.float32)
    got = orc.e4m3_encode_many(y)
    ref = _torch_e4m3(y)
    inrange = y <= 448.0
    assert np.array_equal(got[inrange], ref[inrange])
    assert np.all(got[~inrange] == 0x7E)  # satfinite
    assert (~inrange).sum() > 0 and inrange.sum() + (~inrange).sum() == 31743


def test_e4m3_encode_midpoints_and_neighbours():
    """Every E4M3 midpoint exactly, and one FP32 ulp either side, against torch's RNE cast."""
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    ys = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), vals])
    assert np.array_equal(orc.e4m3_encode_many(ys), _torch_e4m3(ys))
    # above the largest finite value: clamp (torch gives NaN there, so closed form)
    assert list(orc.e4m3_encode_many(np.array([448.0, 463.9, 464.0, 500.0, 1e30], np.float32))) == [0x7E] * 5


def _grid_round(q: np.ndarray) -> np.ndarray:
    """E2M1 rounding of |q| written as piecewise uniform-grid round-half-even (numpy.round):
    spacing 0.5 below 2, 1 in [2, 4), 2 from 4 on, then clamp at 6."""
    q = np.abs(q)
    r = np.where(q < 2, np.round(2 * q) / 2, np.where(q < 4, np.round(q), 2 * np.round(q / 2)))
    return np.minimum(r, 6.0)


MAG_TO_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def test_e2m1_quant_ties_to_even():
    # tie point t*s -> code (RNE: the even code wins): closed form from round-half-even
    expect = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for s in [1.0, 0.5, 448.0, 2.0 ** -9, 1.125, 3.75, 2.0 ** -127]:
        for t, c in expect.items():
            x = np.float32(t * s)
            assert orc.lib().orc_e2m1_quant(float(x), s) == c, (s, t)
            assert orc.lib().orc_e2m1_quant(float(-x), s) == c | 8
            lo = np.nextafter(x, np.float32(0))
            hi = np.nextafter(x, np.float32(1e30))
            if float(lo) / s != t and float(hi) / s != t:
                assert orc.lib().orc_e2m1_quant(float(lo), s) == MAG_TO_CODE[_grid_round(np.array([t - 1e-3]))[0]]
                assert orc.lib().orc_e2m1_quant(float(hi), s) == MAG_TO_CODE[_grid_round(np.array([t + 1e-3]))[0]]


def test_e2m1_quant_all_fp16_times_all_e4m3_scales():
    """8.3M cases: every positive fp16 value against every positive E4M3 scale."""
    scales = torch.arange(1, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    x = np.tile(POS_F16.astype(np.float32), len(scales))
    s = np.repeat(scales, len(POS_F16))
    got = orc.e2m1_quant_many(x, s)
    q = x.astype(np.float64) / s.astype(np.float64)
    ref_mag = _grid_round(q)
    lut = np.zeros(13, np.uint8)
    for m, c in MAG_TO_CODE.items():
        lut[int(m * 2)] = c
    ref = lut[(ref_mag * 2).astype(np.int64)]
    assert np.array_equal(got, ref)
    # sign is the input's, including -0
    assert orc.lib().orc_e2m1_quant(-0.0, 1.0) == 8
    assert orc.lib().orc_e2m1_quant(-1e-9, 1.0) == 8
    assert orc.lib().orc_e2m1_quant(-6.0, 1.0) == 15
    assert orc.lib().orc_e2m1_quant(3.0, 0.0) == 0  # zero scale -> +-0


def test_mx_scale_closed_forms():
    cases = {6.0: 127, 1.0: 125, 7.99: 127, 8.0: 128, 4.0: 127, 3.99: 126, 2.0 ** -30: 95,
             65504.0: 127 + 13, 0.0: 0, 1e-45: 0}
    for amax, byte in cases.items():
        assert orc.lib().orc_mx_scale(amax) == byte, amax


def test_mx_scale_property_all_fp16():
    """OCP rule: amax / 2^X lies in [4, 8) for every positive fp16 amax."""
    xs = POS_F16.astype(np.float64)
    X = np.array([orc.lib().orc_mx_scale(float(a)) for a in POS_F16[::7]], np.int64) - 127
    r = xs[::7] / 2.0 ** X
    assert np.all((r >= 4) & (r < 8))


def test_nv_block_amax_element_gets_code_six():
    """With s = E4M3(amax/6) neither clamped nor underflowed, amax/s is within 6(1 +- 1/16) and
    so always rounds to 6: the scale construction of the [0, 448*6] range."""
    rng = np.random.default_rng(0)
    for _ in range(2000):
        x = (rng.standard_normal(16) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
        codes, sb = orc.quant_block(orc.NVFP4, x)
        s = orc.lib().orc_e4m3_decode(sb)
        if 2.0 ** -6 <= s < 448:
            assert (codes[np.argmax(np.abs(x))] & 7) == 7


def test_mx_block_values_in_grid():
    rng = np.random.default_rng(1)
    for _ in range(500):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        codes, sb = orc.quant_block(orc.MXFP4, x)
        s = 2.0 ** (sb - 127)
        q = x.astype(np.float64) / s
        ref = _grid_round(q) * np.sign(q)
        got = orc.e2m1_table()[codes].astype(np.float64)
        assert np.array_equal(got, ref)


def test_slot_order_from_mfma_layout():
    """The slot order is the key order in which a wave holds S^T after eight 16x16 MFMA
    subtiles: the 16x16 output layout puts rows 4*(lane//16)+i of column lane%16 in lane
    `lane`, so lane group g holds keys 16t + 4g + i of subtile t; flattening (g, t, i) gives
    the slots."""
    expect = []
    for g in range(4):
        for t in range(8):
            for i in range(4):
                expect.append(16 * t + 4 * g + i)
    assert list(orc.slot_tokens()) == expect
    assert sorted(expect) == list(range(128))
