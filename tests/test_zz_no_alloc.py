"""GPU test of sage_fp4_attn_bwd_noalloc, the backward whose workspace is the library's
device-resident array: through the C ABI, its gradients must equal those of sage_fp4_attn_bwd
with a caller-owned workspace bit for bit (same kernels, deterministic), on two calls in a row,
the second with a smaller shape (the array keeps the first call's contents), for NVFP4 and
MXFP4 Q/K, causal or not, fp32 and fp16 gradients. Outputs are prefilled with NaN, so an
unwritten element fails. A shape whose workspace exceeds the array is rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle as orc
from bit_attention_amd import binding as bnd
from helpers import say, to_gpu

pytestmark = pytest.mark.gpu


def _inputs(fmt, B, H, N, D, causal, seed):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, N, D)).astype(np.float16) for _ in range(4))
    Q, K, V = (bnd.quant(to_gpu(x), r, fmt) for x, r in ((q, 0), (k, 1), (v, 2)))
    o = torch.empty((B, H, N, D), dtype=torch.float16, device="cuda")
    lse = torch.empty(B * H * N, dtype=torch.float32, device="cuda")
    bnd.attn_fwd_into(fmt, Q, K, V, (B, H, N, D), o, causal=causal, lse=lse)
    return Q, K, to_gpu(v), o, to_gpu(do), lse


def _grads(shape, dtype):
    return [torch.full(shape, float("nan"), dtype=dtype, device="cuda") for _ in range(3)]


@pytest.mark.parametrize("fmt,causal,dtype", [(orc.NVFP4, True, torch.float32), (orc.MXFP4, False, torch.float16),
                                              (orc.NVFP4, False, torch.float16), (orc.MXFP4, True, torch.float32)])
def test_noalloc_equals_workspace_backward(fmt, causal, dtype):
    for i, (B, H, N, D) in enumerate(((2, 3, 300, 128), (1, 2, 77, 64))):  # the second call is smaller
        say(f"no-alloc backward fmt={fmt} causal={causal} dtype={dtype} shape={(B, H, N, D)} call {i}")
        Q, K, v, o, do, lse = _inputs(fmt, B, H, N, D, causal, 100 * i + fmt)
        ref = _grads((B, H, N, D), dtype)
        ws = bnd.alloc_bwd_workspace(B, H, N, D)
        bnd.attn_bwd_into(fmt, Q, K, v, o, do, lse, *ref, ws, causal=causal)
        got = _grads((B, H, N, D), dtype)
        bnd.attn_bwd_noalloc_into(fmt, Q, K, v, o, do, lse, *got, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.isfinite(b).all(), f"{name}: unwritten or non-finite elements"
            assert torch.equal(a, b), f"{name} differs from the workspace backward"


def test_noalloc_rejects_shapes_beyond_its_array():
    B, H, N, D = 1, 64, 4096, 128
    need = bnd.sage_fp4_attn_bwd_workspace_bytes(B, H, N, D)
    assert need > bnd.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = t.data_ptr()
    rc = bnd.sage_fp4_attn_bwd_noalloc(orc.NVFP4, p, p, p, p, p, p, p, p, B, H, N, D, 0, 0.0, p, p, p,
                                       bnd.OUT_F32, bnd._stream_ptr(None))
    assert bnd.STATUS[rc] == "SAGE_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.count_nonzero(t) == 0  # nothing was launched on the stand-in buffers
