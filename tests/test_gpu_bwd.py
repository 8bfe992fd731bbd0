"""GPU parity of the 8-bit attention backward (sage_fp4_attn_bwd) against the oracle
(oracle/bwd.py).

Both sides get the same O and lse: the oracle forward's output (fp16) and log-sum-exp (fp32),
so the comparison isolates the backward. Each side quantises Q and K for itself (those codes are
bit-exact, checked here too). The bar, per element of dQ, dK and dV:
    |gpu - oracle| <= slack + 1e-4 * mag (+ 2^-11 |oracle| for fp16 outputs)
where the oracle's slack bounds the effect of P and dS codes that lie within float32 rounding of
a rounding boundary and mag is the sum of the magnitudes of the element's terms (float32 sums
and scale products differ from the oracle's float64 by far less than 1e-4 of it).

The workspace the call leaves behind is compared bit-exactly: the bf16 Q^ and K^, the INT8
codes of Q^, K^ and dO with their fp32 scales (slot order undone), and D = rowsum(dO * O) within
float32 rounding.
"""
import numpy as np
import pytest

import oracle as orc
from oracle import bwd as obwd
from bit_attention_amd import synth
from helpers import record_ratio, say, to_gpu

pytestmark = pytest.mark.gpu

SLOT64 = np.array([16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3) for p in range(64)])


def _inputs(fmt, B, H, N, D, causal, wl=1):
    q, k, v = synth.make_qkv(wl, B=B, H=H, N=N, D=D)
    do = synth.make_do(wl, B=B, H=H, N=N, D=D)
    fq = orc.MXFP4 if fmt == orc.MX4_PV8 else fmt
    Q = orc.quant(orc.ROLE_Q, fq, q)
    K = orc.quant(orc.ROLE_K, fq, k)
    V = orc.quant(orc.ROLE_V, fmt, v)
    o, lse = orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), causal=causal, want_lse=True)
    return q, k, v, do, Q, K, o.astype(np.float16), lse.astype(np.float32).reshape(B, H, N)


def _gpu_bwd(fmt, q, k, v, o, do, lse, causal, out_f32=True, keep_ws=False):
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = v.shape
    fq = orc.MXFP4 if fmt == orc.MX4_PV8 else fmt
    Qg = bnd.quant(to_gpu(q), 0, fq)
    Kg = bnd.quant(to_gpu(k), 1, fq)
    dt = torch.float32 if out_f32 else torch.float16
    outs = [torch.full((B, H, N, D), float("nan"), dtype=dt, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    ws.fill_(0xA5)
    bnd.attn_bwd_into(fmt, Qg, Kg, to_gpu(v), to_gpu(o), to_gpu(do), to_gpu(lse), *outs, ws, causal=causal)
    torch.cuda.synchronize()
    res = [t.float().cpu().numpy().astype(np.float64) for t in outs]
    codes = [t.cpu().numpy() for pair in (Qg, Kg) for t in pair]
    return res, codes, (ws.cpu().numpy() if keep_ws else None)


def _check_grads(got, ref, bd, f16_out=False, heads=None):
    names = ("dq", "dk", "dv")
    for t in range(3):
        g, r = got[t], ref[t]
        bound = bd["slack"][t] + 1e-4 * bd["mag"][t] + 1e-30
        if f16_out:
            bound = bound + 2.0 ** -11 * np.abs(r) + 2.0 ** -24
        if heads is not None:
            sel = tuple(np.array(x) for x in zip(*heads))
            g, r, bound = g[sel], r[sel], bound[sel]
        assert np.all(np.isfinite(g)), names[t]
        err = np.abs(g - r)
        worst = float(np.max(err / bound))
        say(f"  {names[t]}: max err {err.max():.3e}, max err/bound {worst:.3f}, max |ref| {np.abs(r).max():.3e}")
        record_ratio(names[t], worst)
        assert worst <= 1.0, names[t]


def _ws_views(ws, B, H, N, D):
    def a256(x):
        return (x + 255) // 256 * 256
    BH, Np = B * H, -(-N // 64) * 64
    nb = Np // 64
    sizes = [BH * N * D * 2] * 2 + [BH * D * Np] * 3 + [BH * D * nb * 4] * 3 + [BH * Np * 4] * 2
    offs = np.cumsum([0] + [a256(s) for s in sizes])
    raw = [ws[offs[i]:offs[i] + sizes[i]] for i in range(len(sizes))]
    bf = [(r.view(np.uint16).astype(np.uint32) << 16).view(np.float32).reshape(B, H, N, D) for r in raw[:2]]
    i8 = [r.view(np.int8).reshape(B, H, D, Np) for r in raw[2:5]]
    sc = [r.view(np.float32).reshape(B, H, nb, D).transpose(0, 1, 3, 2) for r in raw[5:8]]
    dl = raw[8].view(np.float32).reshape(B, H, Np)
    l2 = raw[9].view(np.float32).reshape(B, H, Np)
    return bf, i8, sc, dl, l2


def _mx_table(ws, t, B, H, N, D):
    """The MXFP4 scale table in workspace region t (0: Q, 1: K), [B, H, Np/64, D/32, 16, 4]."""
    Np = -(-N // 64) * 64
    off = 0 if t == 0 else (B * H * N * D * 2 + 255) // 256 * 256
    n = B * H * Np * (D // 32)
    return ws[off:off + n].view(np.uint8).reshape(B, H, Np // 64, D // 32, 16, 4)


def _mx_table_expected(scales, N, D):
    """Byte [b][g][c][s] is the E8M0 scale of token min(64 b + 16 s + c, N - 1), block g."""
    sc = np.asarray(scales).view(np.uint8)
    B, H = sc.shape[:2]
    Np = -(-N // 64) * 64
    tok = np.minimum(np.arange(Np), N - 1)
    t = sc.reshape(B, H, N, D // 32)[:, :, tok, :]                  # [B, H, Np, D/32]
    t = t.reshape(B, H, Np // 64, 4, 16, D // 32)                   # token 64 b + 16 s + c
    return t.transpose(0, 1, 2, 5, 4, 3)                            # [b][g][c][s]


CASES = [
    (orc.NVFP4, 1, 2, 256, 64, False),
    (orc.NVFP4, 2, 2, 200, 128, True),
    (orc.MXFP4, 1, 2, 130, 128, False),
    (orc.MXFP4, 1, 3, 192, 64, True),
    (orc.MX4_PV8, 1, 2, 100, 64, True),
    (orc.NVFP4, 1, 1, 1, 64, False),
    (orc.MXFP4, 1, 1, 65, 128, True),
]


@pytest.mark.parametrize("fmt,B,H,N,D,causal", CASES)
def test_bwd_matches_oracle(fmt, B, H, N, D, causal):
    say(f"bwd parity fmt={fmt} B={B} H={H} N={N} D={D} causal={causal}")
    q, k, v, do, Q, K, o, lse = _inputs(fmt, B, H, N, D, causal)
    got, codes, ws = _gpu_bwd(fmt, q, k, v, o, do, lse, causal, keep_ws=True)
    for a, b in zip(codes, (Q[0], Q[1], K[0], K[1])):
        assert np.array_equal(a.reshape(b.shape), b)
    ref, bd = obwd.attn_bwd(fmt, Q, K, v, o, do, lse, causal=causal, want_bounds=True)
    say(f"  ambiguous codes (dq, dk, dv): {bd['n_amb']}")
    _check_grads(got, ref, bd)

    # the workspace: bf16 Q^, K^ (NVFP4) or the E8M0 scale tables of Q, K (MXFP4); INT8 codes
    # and scales of Q^, K^, dO; D
    fq = orc.MXFP4 if fmt == orc.MX4_PV8 else fmt
    bf, i8, sc, dl, l2 = _ws_views(ws, B, H, N, D)
    xs = (orc.dequant(fq, *Q), orc.dequant(fq, *K), do.astype(np.float64))
    for t in range(2):
        if fq == orc.NVFP4:
            assert np.array_equal(bf[t], xs[t].astype(np.float32))
        else:
            assert np.array_equal(_mx_table(ws, t, B, H, N, D), _mx_table_expected((Q, K)[t][1], N, D))
    for t in range(3):
        for b in range(B):
            for h in range(H):
                codes_o, scales_o = obwd.q8_tokens(xs[t][b, h])
                Np = codes_o.shape[1]
                slots = i8[t][b, h].reshape(D, Np // 64, 64)
                tok = np.empty_like(slots)
                tok[:, :, SLOT64] = slots
                assert np.array_equal(tok.reshape(D, Np).astype(np.int32), codes_o), (t, b, h)
                assert np.array_equal(sc[t][b, h].astype(np.float64), scales_o), (t, b, h)
    dref = np.sum(do.astype(np.float64) * o.astype(np.float64), axis=3)
    gsum = D * 2.0 ** -24 * np.sum(np.abs(do.astype(np.float64) * o.astype(np.float64)), axis=3)
    assert np.all(np.abs(dl[..., :N] - dref) <= gsum + 1e-30)
    assert not dl[..., N:].any() and np.all(l2[..., N:] == np.float32(1e30))
    assert np.array_equal(l2[..., :N], (lse * np.float32(1.4426950408889634)).astype(np.float32))


def test_bwd_fp16_outputs_and_determinism():
    fmt, B, H, N, D, causal = orc.NVFP4, 1, 2, 160, 128, True
    say("bwd fp16 outputs and repeat determinism")
    q, k, v, do, Q, K, o, lse = _inputs(fmt, B, H, N, D, causal)
    ref, bd = obwd.attn_bwd(fmt, Q, K, v, o, do, lse, causal=causal, want_bounds=True)
    got16, _, _ = _gpu_bwd(fmt, q, k, v, o, do, lse, causal, out_f32=False)
    _check_grads(got16, ref, bd, f16_out=True)
    a, _, _ = _gpu_bwd(fmt, q, k, v, o, do, lse, causal)
    b, _, _ = _gpu_bwd(fmt, q, k, v, o, do, lse, causal)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_sm_scale():
    fmt, B, H, N, D, causal = orc.MXFP4, 1, 2, 128, 64, False
    say("bwd with an explicit sm_scale")
    import torch
    from bit_attention_amd import binding as bnd
    q, k, v, do = *synth.make_qkv(1, B=B, H=H, N=N, D=D), synth.make_do(1, B=B, H=H, N=N, D=D)
    Q = orc.quant(0, fmt, q)
    K = orc.quant(1, fmt, k)
    o, lse = orc.attn_fwd(fmt, Q, K, orc.quant(2, fmt, v), (B, H, N, D), sm_scale=0.05, want_lse=True)
    o = o.astype(np.float16)
    lse = lse.astype(np.float32).reshape(B, H, N)
    ref, bd = obwd.attn_bwd(fmt, Q, K, v, o, do, lse, sm_scale=0.05, want_bounds=True)
    Qg, Kg = bnd.quant(to_gpu(q), 0, fmt), bnd.quant(to_gpu(k), 1, fmt)
    outs = [torch.empty((B, H, N, D), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    bnd.attn_bwd_into(fmt, Qg, Kg, to_gpu(v), to_gpu(o), to_gpu(do), to_gpu(lse), *outs, ws, sm_scale=0.05)
    torch.cuda.synchronize()
    _check_grads([t.cpu().numpy().astype(np.float64) for t in outs], ref, bd)


@pytest.mark.parametrize("fmt,causal", [(orc.NVFP4, False), (orc.NVFP4, True), (orc.MXFP4, False),
                                        (orc.MXFP4, True)])
def test_bwd_full_size_sampled_heads(fmt, causal):
    """B4 H32 N4096 D128, the size the benchmark times: every head runs on the GPU with the GPU
    forward's O and lse, except two heads that get the oracle forward's; those two are checked
    against the oracle in full."""
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = 4, 32, 4096, 128
    heads = [(0, 0), (3, 31)]
    flat = [b * H + h for b, h in heads]
    say(f"bwd full size B{B} H{H} N{N} D{D} fmt={fmt} causal={causal}, oracle heads {heads}")
    q, k, v = synth.make_qkv(2)
    do = synth.make_do(2)
    Qg = bnd.quant(to_gpu(q), 0, fmt)
    Kg = bnd.quant(to_gpu(k), 1, fmt)
    Vg = bnd.quant(to_gpu(v), 2, fmt)
    og = torch.empty((B, H, N, D), dtype=torch.float16, device="cuda")
    lg = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(fmt, Qg, Kg, Vg, (B, H, N, D), og, causal=causal, lse=lg)
    # the sampled heads: oracle forward on the oracle's own quantisation
    qs, ks, vs = (x.reshape(B * H, N, D)[flat][None] for x in (q, k, v))
    Qs, Ks, Vs = orc.quant(0, fmt, qs), orc.quant(1, fmt, ks), orc.quant(2, fmt, vs)
    o_s, l_s = orc.attn_fwd(fmt, Qs, Ks, Vs, qs.shape, causal=causal, want_lse=True)
    o_s = o_s.astype(np.float16)
    l_s = l_s.astype(np.float32).reshape(1, len(flat), N)
    for u, (b, h) in enumerate(heads):
        og[b, h] = torch.from_numpy(o_s[0, u]).cuda()
        lg[b, h] = torch.from_numpy(l_s[0, u]).cuda()
    outs = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    bnd.attn_bwd_into(fmt, Qg, Kg, to_gpu(v), og, to_gpu(do), lg, *outs, ws, causal=causal)
    torch.cuda.synchronize()
    got = [t.reshape(B * H, N, D)[flat].cpu().numpy().astype(np.float64)[None] for t in outs]
    for t in outs:
        assert bool(torch.isfinite(t).all())
    dos = do.reshape(B * H, N, D)[flat][None]
    ref, bd = obwd.attn_bwd(fmt, Qs, Ks, vs, o_s, dos, l_s, causal=causal, want_bounds=True)
    say(f"  ambiguous codes (dq, dk, dv): {bd['n_amb']}")
    _check_grads(got, ref, bd)


def test_bwd_stages_equal_full_call():
    """SAGE_BWD_PREP, SAGE_BWD_DKDV, SAGE_BWD_DQ in order give the full call's results bit for bit."""
    import torch
    from bit_attention_amd import binding as bnd
    fmt, B, H, N, D, causal = orc.MXFP4, 1, 2, 300, 128, True
    say("bwd staged calls against the full call")
    q, k, v, do, Q, K, o, lse = _inputs(fmt, B, H, N, D, causal)
    full, _, _ = _gpu_bwd(fmt, q, k, v, o, do, lse, causal)
    Qg, Kg = bnd.quant(to_gpu(q), 0, fmt), bnd.quant(to_gpu(k), 1, fmt)
    outs = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    args = (fmt, Qg, Kg, to_gpu(v), to_gpu(o), to_gpu(do), to_gpu(lse), *outs, ws)
    for stage in (bnd.BWD_PREP, bnd.BWD_DKDV, bnd.BWD_DQ):
        bnd.attn_bwd_into(*args, causal=causal, stage=stage)
    torch.cuda.synchronize()
    for a, b in zip(full, outs):
        assert np.array_equal(a, b.cpu().numpy().astype(np.float64))


def _reference_o_lse(Qh, Kh, V, c, causal, block=2048):
    """Softmax output and row log-sum-exp of one head in float64 (torch on the CPU), over query
    blocks so no N x N array is formed: the exact statistic the forward's log-sum-exp defines,
    used as the backward's O and lse input for both sides."""
    import torch
    Q, K, Vt = (torch.from_numpy(np.ascontiguousarray(x, np.float64)) for x in (Qh, Kh, V))
    N = Q.shape[0]
    O = torch.empty_like(Q[:, :Vt.shape[1]])
    L = torch.empty(N, dtype=torch.float64)
    for i0 in range(0, N, block):
        S = c * (Q[i0:i0 + block] @ K.T)
        if causal:
            rows = torch.arange(i0, min(N, i0 + block))[:, None]
            S = S.masked_fill(torch.arange(N)[None, :] > rows, float("-inf"))
        L[i0:i0 + block] = torch.logsumexp(S, dim=1)
        O[i0:i0 + block] = torch.softmax(S, dim=1) @ Vt
    return O.numpy(), L.numpy()


@pytest.mark.parametrize("wl", [3, 4])
def test_bwd_large_workloads_sampled(wl):
    """Workload 3 (B1 H48 N17776 D64, K with channel offsets) and workload 4 (B1 H32 N32768 D128
    causal, +-20 outliers) at full size: every head runs on the GPU; one head gets a float64
    reference O and lse, and its dK, dV at 192 keys and dQ at 192 queries (first, middle and
    last 64 tokens) are checked against the oracle's sampled mode."""
    import torch
    from bit_attention_amd import binding as bnd
    cfg = synth.WORKLOADS[wl]
    B, H, N, D, causal, fmt = cfg["B"], cfg["H"], cfg["N"], cfg["D"], cfg["causal"], orc.NVFP4
    h = H - 1
    say(f"bwd workload {wl} B{B} H{H} N{N} D{D} causal={causal}, oracle head {h}")
    q, k, v = synth.make_qkv(wl)
    do = synth.make_do(wl)
    Qg, Kg, Vg = bnd.quant(to_gpu(q), 0, fmt), bnd.quant(to_gpu(k), 1, fmt), bnd.quant(to_gpu(v), 2, fmt)
    og = torch.empty((B, H, N, D), dtype=torch.float16, device="cuda")
    lg = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(fmt, Qg, Kg, Vg, (B, H, N, D), og, causal=causal, lse=lg)
    # the checked head: the oracle's quantisation, a float64 reference O and lse
    qs, ks, vs, dos = (x[:, h:h + 1] for x in (q, k, v, do))
    Qs, Ks = orc.quant(0, fmt, qs), orc.quant(1, fmt, ks)
    c = float(np.float32(1.0 / np.sqrt(D)))
    O, L = _reference_o_lse(orc.dequant(fmt, *Qs)[0, 0], orc.dequant(fmt, *Ks)[0, 0],
                            vs[0, 0].astype(np.float64), c, causal)
    o_s = O.astype(np.float16)[None, None]
    l_s = L.astype(np.float32)[None, None]
    og[0, h] = torch.from_numpy(o_s[0, 0]).cuda()
    lg[0, h] = torch.from_numpy(l_s[0, 0]).cuda()
    outs = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    bnd.attn_bwd_into(fmt, Qg, Kg, to_gpu(v), og, to_gpu(do), lg, *outs, ws, causal=causal)
    torch.cuda.synchronize()
    for t in outs:
        assert bool(torch.isfinite(t).all())
    sel = np.concatenate([np.arange(64), np.arange(N // 2 - 32, N // 2 + 32), np.arange(N - 64, N)])
    (rq, rk, rv), bd = obwd.attn_bwd_sampled(fmt, Qs, Ks, vs, o_s, dos, l_s, (0, 0), sel, sel, causal=causal)
    say(f"  ambiguous codes (dq, dk, dv): {bd['n_amb']}")
    got = [outs[t][0, h].cpu().numpy().astype(np.float64)[sel] for t in range(3)]
    _check_grads(got, (rq, rk, rv), dict(slack=bd["slack"], mag=bd["mag"]))


def _random_cases(n=10, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(rng.choice([orc.NVFP4, orc.MXFP4, orc.MX4_PV8])), int(rng.integers(1, 3)),
                    int(rng.integers(1, 4)), int(rng.integers(1, 700)), int(rng.choice([64, 128])),
                    bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("fmt,B,H,N,D,causal,out_f32", _random_cases())
def test_bwd_random_shapes(fmt, B, H, N, D, causal, out_f32):
    """Seeded random shapes, formats, masks and output types; every element checked."""
    say(f"bwd random fmt={fmt} B={B} H={H} N={N} D={D} causal={causal} f32={out_f32}")
    q, k, v, do, Q, K, o, lse = _inputs(fmt, B, H, N, D, causal)
    got, _, _ = _gpu_bwd(fmt, q, k, v, o, do, lse, causal, out_f32=out_f32)
    ref, bd = obwd.attn_bwd(fmt, Q, K, v, o, do, lse, causal=causal, want_bounds=True)
    _check_grads(got, ref, bd, f16_out=not out_f32)


@pytest.mark.parametrize("fmt", [orc.NVFP4, orc.MXFP4])
def test_bwd_most_heads(fmt):
    """B*H = 65535 (the most the C ABI accepts) with a ragged N = 65: two heads, the first and the
    last, get the oracle forward's O and lse and are checked in full."""
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = 1, 65535, 65, 64
    heads = [0, H - 1]
    say(f"bwd limits: fmt={fmt} B*H={H} N={N} D={D}")
    rng = np.random.default_rng(960)
    q, k, v, do = (rng.standard_normal((B, H, N, D), dtype=np.float32).astype(np.float16) for _ in range(4))
    Qg, Kg, Vg = bnd.quant(to_gpu(q), 0, fmt), bnd.quant(to_gpu(k), 1, fmt), bnd.quant(to_gpu(v), 2, fmt)
    og = torch.empty((B, H, N, D), dtype=torch.float16, device="cuda")
    lg = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(fmt, Qg, Kg, Vg, (B, H, N, D), og, lse=lg)
    qs, ks, vs, dos = (x[:, heads] for x in (q, k, v, do))
    Qs, Ks, Vs = orc.quant(0, fmt, qs), orc.quant(1, fmt, ks), orc.quant(2, fmt, vs)
    o_s, l_s = orc.attn_fwd(fmt, Qs, Ks, Vs, qs.shape, want_lse=True)
    o_s = o_s.astype(np.float16)
    l_s = l_s.astype(np.float32).reshape(1, len(heads), N)
    for u, h in enumerate(heads):
        og[0, h] = torch.from_numpy(o_s[0, u]).cuda()
        lg[0, h] = torch.from_numpy(l_s[0, u]).cuda()
    outs = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    bnd.attn_bwd_into(fmt, Qg, Kg, to_gpu(v), og, to_gpu(do), lg, *outs, ws)
    torch.cuda.synchronize()
    for t in outs:
        assert bool(torch.isfinite(t).all())
    got = [t[:, heads].cpu().numpy().astype(np.float64) for t in outs]
    ref, bd = obwd.attn_bwd(fmt, Qs, Ks, vs, o_s, dos, l_s, want_bounds=True)
    _check_grads(got, ref, bd)


@pytest.mark.parametrize("causal,fmt", [(False, orc.NVFP4), (True, orc.NVFP4), (True, orc.MXFP4)])
def test_bwd_longest_sequence(causal, fmt):
    """N = 2^20 (the longest the C ABI accepts), one head, D = 64. The backward is defined for any
    O and lse; at this size both sides get O = V and, per query, the Cauchy-Schwarz bound
    c |Q^_i| max_j |K^_j| + ln N >= the true log-sum-exp (its exact value would take 2^40 dot
    products). dK, dV at 64 keys and dQ at 64 queries (the first and last 32) are checked against
    the oracle's sampled mode; every output must be finite."""
    import torch
    from bit_attention_amd import binding as bnd
    N, D = 1 << 20, 64
    say(f"bwd limits: fmt={fmt} N={N} D={D} causal={causal}")
    rng = np.random.default_rng(970)
    q, k, v, do = (rng.standard_normal((1, 1, N, D), dtype=np.float32).astype(np.float16) for _ in range(4))
    Q, K = orc.quant(0, fmt, q), orc.quant(1, fmt, k)
    Qh, Kh = orc.dequant(fmt, *Q)[0, 0], orc.dequant(fmt, *K)[0, 0]
    c = float(np.float32(1.0 / np.sqrt(D)))
    lse = (c * np.linalg.norm(Qh, axis=1) * np.linalg.norm(Kh, axis=1).max() + np.log(N)).astype(np.float32)
    lse = lse.reshape(1, 1, N)
    Qg, Kg = bnd.quant(to_gpu(q), 0, fmt), bnd.quant(to_gpu(k), 1, fmt)
    outs = [torch.full((1, 1, N, D), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(1, 1, N, D)
    bnd.attn_bwd_into(fmt, Qg, Kg, to_gpu(v), to_gpu(v), to_gpu(do), to_gpu(lse), *outs, ws, causal=causal)
    torch.cuda.synchronize()
    for t in outs:
        assert bool(torch.isfinite(t).all())
    sel = np.concatenate([np.arange(32), np.arange(N - 32, N)])
    (rq, rk, rv), bd = obwd.attn_bwd_sampled(fmt, Q, K, v, v, do, lse, (0, 0), sel, sel, causal=causal)
    got = [outs[t][0, 0].cpu().numpy().astype(np.float64)[sel] for t in range(3)]
    _check_grads(got, (rq, rk, rv), dict(slack=bd["slack"], mag=bd["mag"]))
