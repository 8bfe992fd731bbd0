"""FP64 twin of the oracle's quantised attention: the same algorithm written again here in
float64 numpy, two-pass instead of online, and compared with the oracle's FP32 online version on
the small workloads (B1 H2 N256 D64, NVFP4 and MXFP4, causal or not).

The twin shares only the dequantisation of the stored Q, K, V codes with the oracle (those codecs
are pinned bit-exactly elsewhere). Everything else is re-derived: scores, per-tile maxima, the
two-level P quantisation (E4M3 scales by rounding to three mantissa bits, E8M0 scales by the OCP
exponent rule, E2M1 codes by nearest-grid search with ties to the even code), slot order, the
tile weights exp(t - m) against the row maximum and the normaliser. FP32 and FP64 scores may
round a P decision differently only within the oracle's slack window, so the bar is
|twin - oracle| <= 1e-5 + the oracle's per-row slack."""
import numpy as np
import pytest

import oracle as orc
from bit_attention_amd import synth
from test_oracle_attention import vhat_tokens

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round(y):
    """Nearest E2M1 magnitude to y >= 0 (clamped at 6), ties to the even code index."""
    y = np.minimum(y, 6.0)
    d = np.abs(y[..., None] - E2M1)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    idx = np.where((cand % 2 == 0) & (cand < 99), cand, 99).min(axis=-1)  # an even index among the ties
    idx = np.where(idx == 99, cand.min(axis=-1), idx)
    return E2M1[idx]


def e4m3_round(y):
    """E4M3 value nearest y >= 0, ties to even, clamped to 448 (subnormal step 2^-9)."""
    out = np.zeros_like(y)
    pos = y > 0
    e = np.floor(np.log2(np.where(pos, y, 1.0)))
    step = np.exp2(np.maximum(e, -6.0) - 3.0)
    out = np.where(pos, np.rint(y / step) * step, 0.0)
    return np.minimum(out, 448.0)


def e8m0_scale(amax):
    """The OCP rule 2^(floor(log2 amax) - 2), clamped to [2^-127, 2^127]; 0 for amax == 0."""
    k = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0
    return np.where(amax > 0, np.exp2(np.clip(k, -127, 127)), 0.0)


def twin(fmt, q, k, v, causal):
    B, H, N, D = q.shape
    Q, K, V = (orc.quant(r, fmt, x) for r, x in ((orc.ROLE_Q, q), (orc.ROLE_K, k), (orc.ROLE_V, v)))
    qh, kh = orc.dequant(fmt, *Q), orc.dequant(fmt, *K)
    vh = vhat_tokens(fmt, *V, N)
    c = float(np.float32(1.0 / np.sqrt(D)))
    st = orc.slot_tokens()
    blk = 16 if fmt == orc.NVFP4 else 32
    out = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            x = c * (qh[b, h] @ kh[b, h].T)  # [N, N] float64
            vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
            m = np.where(vis, x, -np.inf).max(axis=1)
            num = np.zeros((N, D)); den = np.zeros(N)
            for t0 in range(0, N, 128):
                keys = t0 + st
                ok = keys < N
                kk = np.where(ok, keys, 0)
                xs = np.where(ok[None, :] & vis[:, kk], x[:, kk], -np.inf)  # [N, 128] slot order
                t = xs.max(axis=1)
                seen = np.isfinite(t)
                E = np.where(np.isfinite(xs), np.exp(xs - np.where(seen, t, 0.0)[:, None]), 0.0)
                P2 = 2688.0 * E if fmt == orc.NVFP4 else E
                Pb = P2.reshape(N, 128 // blk, blk)
                amax = Pb.max(axis=2, keepdims=True)
                s = e4m3_round(amax / 6.0) if fmt == orc.NVFP4 else e8m0_scale(amax)
                Phat = np.where(s > 0, e2m1_round(Pb / np.where(s > 0, s, 1.0)) * s, 0.0).reshape(N, 128)
                w = np.where(seen, np.exp(np.where(seen, t - m, 0.0)), 0.0)
                vt = np.where(ok[:, None], vh[b, h][kk], 0.0)
                num += (w / (2688.0 if fmt == orc.NVFP4 else 1.0))[:, None] * (Phat @ vt)
                den += w * E.sum(axis=1)
            out[b, h] = num / den[:, None]
    return out, (Q, K, V)


@pytest.mark.parametrize("wl", [1, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_fp64_twin_agrees_with_oracle(wl, causal):
    fmt = orc.MXFP4 if wl == 5 else orc.NVFP4
    q, k, v = synth.make_qkv(wl)
    B, H, N, D = q.shape
    ref, (Q, K, V) = twin(fmt, q, k, v, causal)
    got, slack = orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), causal=causal, want_slack=True)
    err = np.abs(got.astype(np.float64) - ref).reshape(-1, D).max(axis=1)
    assert np.all(err <= 1e-5 + slack), f"max err {err.max()} (rows with slack: {(slack > 0).sum()})"
    assert np.median(err) < 1e-6
