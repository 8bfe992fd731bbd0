"""Host tests of the torch wrappers' argument checks: the C ABI cannot see buffer sizes, so the
wrappers must reject undersized, non-contiguous or mis-typed buffers before any launch. The
tests run on the CPU: CPU tensors stand in for device tensors (the device predicate is patched)
and every raw entry point that would launch is replaced by one that fails the test if reached.
The size queries go to the built library, which needs no GPU."""
import pytest
import torch

from bit_attention_amd import binding as bnd

LAUNCHING = ["sage_fp4_quant", "sage_fp4_attn_fwd", "sage_fp4_attn_fwd_direct_p", "sage_fp4_attn_fwd_lse",
             "sage_fp4_attn_bwd", "sage_fp4_attn_bwd_stage", "sage_fp4_kv16_prep", "sage_fp4_quant_kv16",
             "sage_fp4_attn_fwd_kv16"]


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    monkeypatch.setattr(bnd, "_on_gpu", lambda t: True)
    for name in LAUNCHING:
        monkeypatch.setattr(bnd, name, lambda *a, _n=name: pytest.fail(f"{_n} was reached"))
    monkeypatch.setattr(bnd, "_stream_ptr", lambda s: None)


SHAPE = (1, 2, 200, 64)


def _pair(role, fmt=bnd.NVFP4, shrink=0):
    nc, ns = bnd._sizes(role, fmt, *SHAPE)
    return torch.zeros(nc - shrink, dtype=torch.uint8), torch.zeros(ns, dtype=torch.uint8)


def test_quant_rejects_short_codes_and_scales():
    x = torch.zeros(SHAPE, dtype=torch.float16)
    for role in (bnd.ROLE_Q, bnd.ROLE_K, bnd.ROLE_V):
        c, s = _pair(role, shrink=1)
        with pytest.raises(ValueError, match="codes"):
            bnd.quant_into(x, role, bnd.NVFP4, c, s)
        c, s = _pair(role)
        with pytest.raises(ValueError, match="scales"):
            bnd.quant_into(x, role, bnd.NVFP4, c, s[:-1])
    with pytest.raises(TypeError):
        bnd.quant_into(x.float(), bnd.ROLE_Q, bnd.NVFP4, *_pair(bnd.ROLE_Q))


def test_attn_fwd_rejects_bad_out_and_operands():
    q, k, v = _pair(bnd.ROLE_Q), _pair(bnd.ROLE_K), _pair(bnd.ROLE_V)
    B, H, N, D = SHAPE
    with pytest.raises(ValueError, match="exactly"):
        bnd.attn_fwd_into(bnd.NVFP4, q, k, v, SHAPE, torch.zeros(B * H * N * D - 1))
    with pytest.raises(TypeError, match="contiguous"):
        bnd.attn_fwd_into(bnd.NVFP4, q, k, v, SHAPE, torch.zeros(B, H, D, N).transpose(2, 3))
    with pytest.raises(ValueError, match="v codes"):
        bnd.attn_fwd_into(bnd.NVFP4, q, k, _pair(bnd.ROLE_V, shrink=16), SHAPE, torch.zeros(SHAPE))
    # V's padded layout: MXFP4 codes of Q are enough bytes for Q but not for V
    with pytest.raises(ValueError):
        bnd.attn_fwd_into(bnd.NVFP4, q, k, q, SHAPE, torch.zeros(SHAPE))
    with pytest.raises(ValueError, match="lse"):
        bnd.attn_fwd_into(bnd.NVFP4, q, k, v, SHAPE, torch.zeros(SHAPE), lse=torch.zeros(B * H * N + 1))
    with pytest.raises(TypeError):
        bnd.attn_fwd_into(bnd.NVFP4, q, k, v, SHAPE, torch.zeros(SHAPE, dtype=torch.float64))


def test_attn_bwd_rejects_small_workspace_and_bad_gradients():
    q, k = _pair(bnd.ROLE_Q), _pair(bnd.ROLE_K)
    B, H, N, D = SHAPE
    v, o, do = (torch.zeros(SHAPE, dtype=torch.float16) for _ in range(3))
    lse = torch.zeros(B * H * N)
    grads = [torch.zeros(SHAPE) for _ in range(3)]
    need = bnd.sage_fp4_attn_bwd_workspace_bytes(*SHAPE)
    with pytest.raises(ValueError, match="workspace"):
        bnd.attn_bwd_into(bnd.NVFP4, q, k, v, o, do, lse, *grads, torch.zeros(need - 1, dtype=torch.uint8))
    ws = torch.zeros(need, dtype=torch.uint8)
    with pytest.raises(ValueError, match="dk"):
        bnd.attn_bwd_into(bnd.NVFP4, q, k, v, o, do, lse, grads[0], torch.zeros(B, H, N, D - 1), grads[2], ws)
    with pytest.raises(TypeError, match="dv"):
        bnd.attn_bwd_into(bnd.NVFP4, q, k, v, o, do, lse, grads[0], grads[1], grads[2].half(), ws)
    with pytest.raises(ValueError, match="lse"):
        bnd.attn_bwd_into(bnd.NVFP4, q, k, v, o, do, lse[:-1], *grads, ws)
    with pytest.raises(ValueError, match="q codes"):
        bnd.attn_bwd_into(bnd.NVFP4, _pair(bnd.ROLE_Q, shrink=1), k, v, o, do, lse, *grads, ws)


def test_kv16_wrappers_reject_short_buffers_and_bad_roles():
    B, H, N, D = SHAPE
    need = bnd.sage_fp4_kv16_bytes(*SHAPE)
    k, v = _pair(bnd.ROLE_K), _pair(bnd.ROLE_V)
    with pytest.raises(ValueError, match="kv16"):
        bnd.kv16_prep(k, v, SHAPE, torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="v codes"):
        bnd.kv16_prep(k, _pair(bnd.ROLE_V, shrink=16), SHAPE, torch.zeros(need, dtype=torch.uint8))
    x = torch.zeros(SHAPE, dtype=torch.float16)
    kv = torch.zeros(need, dtype=torch.uint8)
    with pytest.raises(ValueError, match="role"):
        bnd.quant_kv16_into(x, bnd.ROLE_Q, *_pair(bnd.ROLE_Q), kv)
    with pytest.raises(ValueError, match="kv16"):
        bnd.quant_kv16_into(x, bnd.ROLE_K, *k, kv[:-1])
    with pytest.raises(ValueError, match="codes"):
        bnd.quant_kv16_into(x, bnd.ROLE_V, *_pair(bnd.ROLE_V, shrink=1), kv)
    with pytest.raises(TypeError):
        bnd.quant_kv16_into(x.float(), bnd.ROLE_K, *k, kv)
    with pytest.raises(ValueError, match="shape"):
        bnd.quant_kv16(x, torch.zeros(B, H, N + 1, D, dtype=torch.float16), kv16=kv)
    q = _pair(bnd.ROLE_Q)
    with pytest.raises(ValueError, match="kv16"):
        bnd.attn_fwd_kv16_into(q, kv[:-1], SHAPE, torch.zeros(SHAPE))
    with pytest.raises(ValueError, match="exactly"):
        bnd.attn_fwd_kv16_into(q, kv, SHAPE, torch.zeros(B * H * N * D - 1))
    with pytest.raises(ValueError, match="lse"):
        bnd.attn_fwd_kv16_into(q, kv, SHAPE, torch.zeros(SHAPE), lse=torch.zeros(B * H * N - 1))
