"""Shared helpers for the GPU tests: run the HIP path through the C ABI and the oracle on the same
seeded inputs (each side quantises for itself; nothing flows from one to the other)."""
import os
import sys

import numpy as np

import oracle as orc
from bit_attention_amd import synth

_CACHE = {}


# worst |gpu - oracle| / bound of each test that checks against a bound, by test id; the
# session's terminal summary prints them (tests/conftest.py)
BOUND_RATIOS = {}


def record_ratio(what, ratio):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    key = f"{test} {what}"
    BOUND_RATIOS[key] = max(BOUND_RATIOS.get(key, 0.0), float(ratio))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workload(wl, **kw):
    key = (wl, tuple(sorted((k, tuple(v) if isinstance(v, list) else v) for k, v in kw.items())))
    if key not in _CACHE:
        if len(_CACHE) > 2:
            _CACHE.clear()
        _CACHE[key] = synth.make_qkv(wl, **kw)
    return _CACHE[key]


def to_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_quant(x, role, fmt):
    """numpy fp16 [B,H,N,D] -> numpy (codes, scales) in the oracle's array shapes."""
    from bit_attention_amd import binding as bnd
    B, H, N, D = x.shape
    c, s = bnd.quant(to_gpu(x), role, fmt)
    import torch
    torch.cuda.synchronize()
    blk = 16 if fmt == 0 else 32
    if role == 2:
        Np = orc.padded_n(N)
        vb = 128 if fmt == 2 else 64
        return c.cpu().numpy().reshape(B, H, Np // 128, D, vb), s.cpu().numpy().reshape(B, H, Np // 128, D, 128 // blk)
    return c.cpu().numpy().reshape(B, H, N, D // 2), s.cpu().numpy().reshape(B, H, N, D // blk)


def gpu_attn(fmt, q, k, v, causal, out_f32=True, prefill_nan=True, direct_p=False):
    """Full HIP path on numpy fp16 inputs: three quant launches + one attention launch
    (sage_fp4_attn_fwd, or sage_fp4_attn_fwd_direct_p when direct_p)."""
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = q.shape
    Q = bnd.quant(to_gpu(q), 0, fmt)
    K = bnd.quant(to_gpu(k), 1, fmt)
    V = bnd.quant(to_gpu(v), 2, fmt)
    out = torch.empty((B, H, N, D), dtype=torch.float32 if out_f32 else torch.float16, device="cuda")
    if prefill_nan:
        out.fill_(float("nan"))
    bnd.attn_fwd_into(fmt, Q, K, V, (B, H, N, D), out, causal=causal, direct_p=direct_p)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_attn(fmt, q, k, v, causal, rows=None, direct_p=False):
    """Oracle on its own quantisation of the same inputs; returns (out, slack)."""
    B, H, N, D = q.shape
    Q = orc.quant(orc.ROLE_Q, fmt, q)
    K = orc.quant(orc.ROLE_K, fmt, k)
    V = orc.quant(orc.ROLE_V, fmt, v)
    return orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), causal=causal, rows=rows, want_slack=True,
                        direct_p=direct_p)


def sample_rows(N, n_each=8, seed=0):
    """Query rows: the first and last tiles' edges, tile boundaries and a few random ones."""
    rng = np.random.default_rng(seed)
    r = set(range(min(n_each, N)))
    r |= set(range(max(0, N - n_each), N))
    for b in (127, 128, 129, 255, 256):
        if b < N:
            r.add(b)
    r |= set(int(x) for x in rng.integers(0, N, n_each))
    return np.array(sorted(r), np.int64)


TOL = 2e-3  # max-abs output tolerance against the oracle


def compare(gpu_rows, orc_rows, slack, what, use_slack=False, extra=None):
    """Every row: |gpu - oracle| <= TOL (plus `extra`, a per-row bound the caller documents, such
    as the rounding of an fp16 output). With use_slack, also plus the oracle's per-row slack: only
    the tests whose inputs push P decisions onto their boundaries (scores far outside the
    workloads' range) use it, and each says why. The slack is always reported."""
    err = np.abs(gpu_rows.astype(np.float64) - orc_rows.astype(np.float64)).max(axis=-1)
    bound = TOL + (extra if extra is not None else 0.0) + (slack if use_slack else 0.0)
    bad = np.nonzero(~(err <= bound))[0]
    clean = slack == 0
    stats = dict(max_err=float(err.max()), max_err_clean=float(err[clean].max()) if clean.any() else 0.0,
                 rows=int(err.size), rows_with_slack=int((~clean).sum()), max_slack=float(slack.max()),
                 bar="2e-3 + slack" if use_slack else "2e-3")
    say(f"  [{what}] {stats}")
    assert bad.size == 0, (f"{what}: {bad.size} rows beyond the bar, worst row {bad[np.argmax(err[bad])]} "
                           f"err {err[bad].max()} slack {slack[bad].max()}")
    return stats
