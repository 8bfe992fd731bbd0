"""GPU parity of the NVFP4 path with K and V dequantised once (sage_fp4_kv16_prep, then
sage_fp4_attn_fwd_kv16) through the C ABI.

- The prep's buffer holds exactly the oracle's own dequantisation of the same inputs: K-hat
  value for value, rows past N zero; V-hat in the tile-major slot order, padding zero.
- The attention from the buffer equals sage_fp4_attn_fwd on the same codes bit for bit (fp32 and
  fp16 outputs, and lse against sage_fp4_attn_fwd_lse), at small and ragged shapes and at the full
  workload sizes bench.py times.
- Against the oracle directly, every row of small shapes within 2e-3 (the bar of
  tests/test_gpu_attn.py; the slack is reported, not added).
- Equal to the codes path at the C ABI's limits too: N = 2^20, and B*H = 65535.
- A buffer smaller than sage_fp4_kv16_bytes is refused before any launch.
- sage_fp4_quant_kv16 (K or V quantised with its half of the buffer in the same pass) writes the
  codes and scales of sage_fp4_quant and the buffer bytes of sage_fp4_kv16_prep, byte for byte,
  every byte of each (outputs pre-filled), and leaves the other role's half as it was."""
import numpy as np
import pytest

import oracle as orc
from helpers import compare, oracle_attn, say, to_gpu, workload

pytestmark = pytest.mark.gpu

NV = orc.NVFP4


def _quant_all(q, k, v):
    from bit_attention_amd import binding as bnd
    return tuple(bnd.quant(to_gpu(x), r, NV) for x, r in ((q, 0), (k, 1), (v, 2)))


def _both(Q, K, V, shape, causal, out_f32=True, with_lse=False):
    """(codes-path out, kv16-path out[, lse of each]) on the same quantised operands."""
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = shape
    dt = torch.float32 if out_f32 else torch.float16
    kv = bnd.kv16_prep(K, V, shape)
    o1 = torch.full(shape, float("nan"), dtype=dt, device="cuda")
    o2 = torch.full(shape, float("nan"), dtype=dt, device="cuda")
    l1 = l2 = None
    if with_lse:
        l1 = torch.full((B * H * N,), float("nan"), dtype=torch.float32, device="cuda")
        l2 = torch.full((B * H * N,), float("nan"), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(NV, Q, K, V, shape, o1, causal=causal, lse=l1)
    bnd.attn_fwd_kv16_into(Q, kv, shape, o2, causal=causal, lse=l2)
    torch.cuda.synchronize()
    res = [o1.float().cpu().numpy(), o2.float().cpu().numpy()]
    if with_lse:
        res += [l1.cpu().numpy(), l2.cpu().numpy()]
    return res


def _bit_equal(a, b, what):
    assert a.dtype == np.float32 and b.dtype == np.float32
    assert np.all(np.isfinite(b)), f"{what}: unwritten or non-finite values"
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
        f"{what}: differs from sage_fp4_attn_fwd, max |diff| {np.abs(a - b).max()}"


PREP = [(1, 2, 300, 128), (2, 3, 129, 64), (1, 1, 1, 128), (1, 2, 256, 64), (1, 1, 640, 128)]


@pytest.mark.parametrize("shape", PREP)
def test_prep_equals_oracle_dequantisation(shape):
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = shape
    Np = orc.padded_n(N)
    q, k, v = workload(3, B=B, H=H, N=N, D=D)
    say(f"kv16 prep shape={shape}")
    K = bnd.quant(to_gpu(k), 1, NV)
    V = bnd.quant(to_gpu(v), 2, NV)
    kv = bnd.kv16_prep(K, V, shape)
    torch.cuda.synchronize()
    h = kv.cpu().numpy().view(np.float16).astype(np.float64)
    kh = h[:B * H * Np * D].reshape(B, H, Np, D)
    vh = h[B * H * Np * D:2 * B * H * Np * D].reshape(B, H, Np // 128, D, 128)
    Ko = orc.quant(orc.ROLE_K, NV, k)
    Vo = orc.quant(orc.ROLE_V, NV, v)
    assert np.array_equal(kh[:, :, :N], orc.dequant(NV, *Ko)), "K-hat"
    assert np.all(kh[:, :, N:] == 0), "K-hat rows past N"
    vrows = np.ascontiguousarray(np.transpose(vh, (0, 1, 3, 2, 4))).reshape(B, H, D, Np)
    assert np.array_equal(vrows, orc.dequant(NV, *orc.v_by_channel(*Vo))), "V-hat"


SMALL = [((1, 2, 256, 64), 1), ((1, 2, 300, 128), 1), ((2, 3, 129, 64), 1), ((1, 1, 1, 128), 1),
         ((1, 2, 127, 64), 1), ((1, 1, 640, 128), 2)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,wl", SMALL)
def test_small_equal_to_codes_path_and_oracle(causal, shape, wl):
    B, H, N, D = shape
    q, k, v = workload(wl, B=B, H=H, N=N, D=D)
    say(f"kv16 attn causal={causal} shape={shape}")
    Q, K, V = _quant_all(q, k, v)
    a, b, la, lb = _both(Q, K, V, shape, causal, with_lse=True)
    _bit_equal(a, b, f"out {shape}")
    _bit_equal(la, lb, f"lse {shape}")
    o, sl = oracle_attn(NV, q, k, v, causal)
    compare(b.reshape(-1, D), o.reshape(-1, D), sl, f"kv16 causal{causal} {shape}")


@pytest.mark.parametrize("wl,causal", [(2, False), (2, True), (3, False), (3, True), (4, True)])
def test_full_size_equal_to_codes_path(wl, causal):
    q, k, v = workload(wl)
    shape = q.shape
    say(f"kv16 full workload {wl} causal={causal} shape={shape}")
    Q, K, V = _quant_all(q, k, v)
    a, b = _both(Q, K, V, shape, causal)
    _bit_equal(a, b, f"workload {wl} causal {causal}")


def test_fp16_output_equal_to_codes_path():
    q, k, v = workload(1, B=1, H=3, N=1000, D=128)
    Q, K, V = _quant_all(q, k, v)
    a, b = _both(Q, K, V, q.shape, True, out_f32=False)
    _bit_equal(a, b, "fp16 output")


def test_one_buffer_serves_two_calls():
    """The buffer is read-only for the attention: two calls (different masks) from one prep equal
    the codes path each time."""
    import torch
    from bit_attention_amd import binding as bnd
    q, k, v = workload(1, B=2, H=2, N=700, D=64)
    shape = q.shape
    Q, K, V = _quant_all(q, k, v)
    kv = bnd.kv16_prep(K, V, shape)
    for causal in (True, False):
        o1 = torch.empty(shape, dtype=torch.float32, device="cuda")
        o2 = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        bnd.attn_fwd_into(NV, Q, K, V, shape, o1, causal=causal)
        bnd.attn_fwd_kv16_into(Q, kv, shape, o2, causal=causal)
        torch.cuda.synchronize()
        _bit_equal(o1.cpu().numpy(), o2.cpu().numpy(), f"reuse causal {causal}")


def test_small_buffer_refused_before_launch():
    import ctypes as C
    import torch
    from bit_attention_amd import binding as bnd
    q, k, v = workload(1, B=1, H=1, N=200, D=64)
    shape = q.shape
    Q, K, V = _quant_all(q, k, v)
    need = bnd.sage_fp4_kv16_bytes(*shape)
    kv = torch.full((need,), 0x7B, dtype=torch.uint8, device="cuda")
    ptrs = [C.c_void_p(t.data_ptr()) for pair in (K, V) for t in pair]
    assert bnd.sage_fp4_kv16_prep(*ptrs, *shape, C.c_void_p(kv.data_ptr()), need - 1, None) == -7
    out = torch.full(shape, 5.0, dtype=torch.float32, device="cuda")
    assert bnd.sage_fp4_attn_fwd_kv16(C.c_void_p(Q[0].data_ptr()), C.c_void_p(Q[1].data_ptr()),
                                      C.c_void_p(kv.data_ptr()), need - 1, *shape, 0, 0.0,
                                      C.c_void_p(out.data_ptr()), 1, None, None) == -7
    torch.cuda.synchronize()
    assert bool((kv == 0x7B).all()) and bool((out == 5.0).all()), "nothing may be written"


@pytest.mark.parametrize("shape", [(1, 1, 1 << 20, 64), (1, 65535, 1, 128)])
def test_limits_equal_to_codes_path(shape):
    """The longest sequence and the most heads the C ABI accepts (the prep's largest grids in x and
    in y): equal to the codes path, which tests/test_gpu_limits.py checks against the oracle."""
    rng = np.random.default_rng(990)
    q, k, v = (rng.standard_normal(shape).astype(np.float16) for _ in range(3))
    Q, K, V = _quant_all(q, k, v)
    for causal in ((False, True) if shape[2] > 1 else (False,)):
        say(f"kv16 limits shape={shape} causal={causal}")
        a, b = _both(Q, K, V, shape, causal)
        _bit_equal(a, b, f"limits {shape} causal {causal}")


FUSED = [(1, 2, 300, 128), (2, 3, 129, 64), (1, 1, 1, 128), (1, 2, 256, 64), (1, 1, 640, 128), (3, 1, 1000, 64)]


def _fused_equals_separate(k, v, what):
    """quant_kv16 on pre-filled buffers against quant + kv16_prep, byte for byte."""
    import torch
    from bit_attention_amd import binding as bnd
    B, H, N, D = k.shape
    need = bnd.sage_fp4_kv16_bytes(B, H, N, D)
    K = bnd.quant(k, 1, NV)
    V = bnd.quant(v, 2, NV)
    ref = bnd.kv16_prep(K, V, k.shape)
    kv = torch.full((need,), 0x7B, dtype=torch.uint8, device="cuda")
    Kf, Vf, kv = bnd.quant_kv16(k, v, kv16=kv)
    torch.cuda.synchronize()
    for (a, b), name in (((K[0], Kf[0]), "K codes"), ((K[1], Kf[1]), "K scales"), ((V[0], Vf[0]), "V codes"),
                         ((V[1], Vf[1]), "V scales"), ((ref, kv), "kv16 buffer")):
        assert torch.equal(a, b), f"{what}: {name} differ at {int((a != b).sum())} bytes"


@pytest.mark.parametrize("shape", FUSED)
def test_quant_kv16_equals_quant_and_prep(shape):
    import torch
    B, H, N, D = shape
    q, k, v = workload(3, B=B, H=H, N=N, D=D)
    say(f"quant_kv16 shape={shape}")
    _fused_equals_separate(to_gpu(k), to_gpu(v), f"shape {shape}")


@pytest.mark.parametrize("wl", [2, 3, 4])
def test_quant_kv16_full_size(wl):
    q, k, v = workload(wl)
    say(f"quant_kv16 full workload {wl} shape={q.shape}")
    _fused_equals_separate(to_gpu(k), to_gpu(v), f"workload {wl}")


@pytest.mark.parametrize("shape", [(1, 1, 1 << 20, 64), (1, 65535, 1, 128)])
def test_quant_kv16_limits(shape):
    """The K-hat grid's largest x (N = 2^20) and y (B*H = 65535) extents."""
    rng = np.random.default_rng(991)
    k, v = (to_gpu(rng.standard_normal(shape).astype(np.float16)) for _ in range(2))
    say(f"quant_kv16 limits shape={shape}")
    _fused_equals_separate(k, v, f"limits {shape}")


def test_quant_kv16_one_role_leaves_other_half():
    import ctypes as C
    import torch
    from bit_attention_amd import binding as bnd
    shape = (2, 2, 300, 64)
    B, H, N, D = shape
    q, k, v = workload(1, B=B, H=H, N=N, D=D)
    need = bnd.sage_fp4_kv16_bytes(*shape)
    half = need // 2
    for role, x, written in ((1, k, slice(0, half)), (2, v, slice(half, need))):
        kv = torch.full((need,), 0x7B, dtype=torch.uint8, device="cuda")
        codes, scales = bnd.alloc_quant(role, NV, *shape)
        xg = to_gpu(x)
        rc = bnd.sage_fp4_quant_kv16(role, C.c_void_p(xg.data_ptr()), *shape, C.c_void_p(codes.data_ptr()),
                                     C.c_void_p(scales.data_ptr()), C.c_void_p(kv.data_ptr()), need, None)
        assert rc == 0
        torch.cuda.synchronize()
        untouched = torch.ones(need, dtype=torch.bool, device="cuda")
        untouched[written] = False
        assert bool((kv[untouched] == 0x7B).all()), f"role {role} wrote outside its half"
        assert not bool((kv[written] == 0x7B).all()), f"role {role} wrote nothing"


@pytest.mark.parametrize("causal", [False, True])
def test_attention_from_quant_kv16_equals_codes_path(causal):
    """The whole fused path (Q quantised as usual, K and V with their halves of the buffer, then
    the attention from the buffer) against the codes path, bit for bit."""
    import torch
    from bit_attention_amd import binding as bnd
    q, k, v = workload(2, B=1, H=4, N=1000, D=128)
    shape = q.shape
    say(f"quant_kv16 + attention causal={causal}")
    Q = bnd.quant(to_gpu(q), 0, NV)
    K, V, kv = bnd.quant_kv16(to_gpu(k), to_gpu(v))
    o1 = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    o2 = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(NV, Q, K, V, shape, o1, causal=causal)
    bnd.attn_fwd_kv16_into(Q, kv, shape, o2, causal=causal)
    torch.cuda.synchronize()
    _bit_equal(o1.cpu().numpy(), o2.cpu().numpy(), f"fused path causal {causal}")
