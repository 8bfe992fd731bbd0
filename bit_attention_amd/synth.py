"""Seeded synthetic inputs for the attention workloads (shared by the tests, the benchmark and the
smoke check; holds none of the attention or quantisation arithmetic).

Generator: counter-based SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; the finaliser constants of Vigna's splitmix64.c), uniform doubles from
the top 53 bits, standard normals by the Box-Muller transform, rounded to fp16 (round to nearest
even). Element i of stream `seed` is mix(seed + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64), so any
sub-range can be generated independently of numpy's or torch's own generators.

Workloads (seed = 1000 * workload + tensor id; Q=0, K=1, V=2, channel offsets=3, dO=4,
outlier mask = 10 + tensor, outlier sign = 20 + tensor):
  1 tiny:      B=1 H=2  N=256   D=64,  Q,K,V ~ N(0,1)
  2 sweep:     B=4 H=32 N=4096  D=128 (N also 1024..16384), Q,K,V ~ N(0,1)
  3 video-DiT: B=1 H=48 N=17776 D=64,  K = N(0,1) + o[h,d], o ~ N(0, sd=3) per (head, channel)
  4 long LLM:  B=1 H=32 N=32768 D=128 causal, Q,K,V ~ N(0,1), each entry replaced with
               probability 0.001 by +-20 (fair sign)
  5 MXFP4:     the data of workload 1
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def bits(seed: int, start: int, n: int) -> np.ndarray:
    """SplitMix64 outputs for counters start..start+n-1 of stream `seed`."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        return _mix(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GAMMA)


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Doubles in [0, 1)."""
    return (bits(seed, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _normal_f64(seed: int, start: int, m: int) -> np.ndarray:
    """Normals start..start+m-1 of stream `seed` (start even); pair k uses uniforms 2k, 2k+1."""
    assert start % 2 == 0
    npair = (m + 1) // 2
    u = uniform(seed, 2 * npair, start=start)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    z = np.empty(2 * npair, np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return z[:m]


def normal(seed: int, n: int) -> np.ndarray:
    """n standard normals (float64)."""
    out = np.empty(n, np.float64)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = _normal_f64(seed, s, m)
    return out


def normal_f16(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Normals start..start+n-1 of stream `seed`, rounded to float16."""
    out = np.empty(n, np.float16)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = _normal_f64(seed, start + s, m).astype(np.float16)
    return out


WORKLOADS = {
    1: dict(B=1, H=2, N=256, D=64, causal=False, fmt="nvfp4", name="tiny"),
    2: dict(B=4, H=32, N=4096, D=128, causal=False, fmt="nvfp4", name="sweep"),
    3: dict(B=1, H=48, N=17776, D=64, causal=False, fmt="nvfp4", name="video_dit"),
    4: dict(B=1, H=32, N=32768, D=128, causal=True, fmt="nvfp4", name="long_causal"),
    5: dict(B=1, H=2, N=256, D=64, causal=False, fmt="mxfp4", name="tiny_mxfp4"),
}


def _outliers(flat: np.ndarray, wl: int, tid: int, start: int) -> None:
    """Replace entries with probability 0.001 by +-20 (fair sign), in place; `flat` holds
    elements start..start+len-1 of the tensor."""
    n = flat.size
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        hit = uniform(1000 * wl + 10 + tid, m, start=start + s) < 0.001
        sign = uniform(1000 * wl + 20 + tid, m, start=start + s) < 0.5
        idx = np.nonzero(hit)[0]
        flat[s + idx] = np.where(sign[idx], np.float16(-20.0), np.float16(20.0))


def make_qkv(wl: int, B=None, H=None, N=None, D=None, heads=None):
    """Q, K, V float16 [B,H,N,D] of workload `wl` (sizes overridable, e.g. for the N sweep).

    heads: optional list of flat (b*H + h) indices; only those heads are generated and the
    result has shape [1, len(heads), N, D], equal to the matching slices of the full tensors."""
    base = 1 if wl == 5 else wl
    cfg = WORKLOADS[wl]
    B = B or cfg["B"]; H = H or cfg["H"]; N = N or cfg["N"]; D = D or cfg["D"]
    hs = list(range(B * H)) if heads is None else [int(h) for h in heads]
    per = N * D
    offs = None
    if base == 3:
        # channel offsets o[h, d] ~ N(0, sd=3), shared by all tokens of a head
        offs = 3.0 * normal(1000 * base + 3, H * D).reshape(H, D)
    out = []
    for tid in range(3):
        seed = 1000 * base + tid
        x = np.empty((len(hs), N, D), np.float16)
        for u, bh in enumerate(hs):
            flat = normal_f16(seed, per, start=bh * per)
            if offs is not None and tid == 1:
                flat = (flat.astype(np.float64).reshape(N, D) + offs[bh % H][None, :]).astype(np.float16).reshape(-1)
            if base == 4:
                _outliers(flat, base, tid, bh * per)
            x[u] = flat.reshape(N, D)
        out.append(x.reshape(B, H, N, D) if heads is None else x.reshape(1, len(hs), N, D))
    return tuple(out)


def make_do(wl: int, B=None, H=None, N=None, D=None, heads=None):
    """The output gradient dO ~ N(0,1), float16 [B,H,N,D], of workload `wl` (stream id 4; the
    same head slicing as make_qkv)."""
    base = 1 if wl == 5 else wl
    cfg = WORKLOADS[wl]
    B = B or cfg["B"]; H = H or cfg["H"]; N = N or cfg["N"]; D = D or cfg["D"]
    hs = list(range(B * H)) if heads is None else [int(h) for h in heads]
    per = N * D
    x = np.empty((len(hs), N, D), np.float16)
    for u, bh in enumerate(hs):
        x[u] = normal_f16(1000 * base + 4, per, start=bh * per).reshape(N, D)
    return x.reshape(B, H, N, D) if heads is None else x.reshape(1, len(hs), N, D)
