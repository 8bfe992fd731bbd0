"""The entry points inside a HIP graph: one step (three sage_fp4_quant launches and one attention
launch; with the kv16 path also sage_fp4_kv16_prep; in the training form also the backward's five
launches) captured with torch.cuda.CUDAGraph and replayed several times, with eager work and
synchronisations between the replays that change the inputs, must give exactly the eager results
every time. The library
allocates nothing, synchronises nothing and issues no memset, so each launch is one kernel node."""
import numpy as np
import pytest
import torch

from bit_attention_amd import binding as bnd
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,direct_p,causal", [(bnd.NVFP4, False, False), (bnd.NVFP4, False, True),
                                                 (bnd.MXFP4, True, False), (bnd.MX4_PV8, False, True)])
def test_graph_replays_match_eager(fmt, direct_p, causal):
    B, H, N, D = 2, 4, 640, 128
    shape = (B, H, N, D)
    g = torch.Generator(device="cuda").manual_seed(11)
    q, k, v = (torch.randn(shape, generator=g, device="cuda").half() for _ in range(3))
    Q, K, V = (bnd.alloc_quant(r, fmt, *shape) for r in (bnd.ROLE_Q, bnd.ROLE_K, bnd.ROLE_V))
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(B * H * N, dtype=torch.float32, device="cuda")

    def step():
        bnd.quant_into(q, bnd.ROLE_Q, fmt, *Q)
        bnd.quant_into(k, bnd.ROLE_K, fmt, *K)
        bnd.quant_into(v, bnd.ROLE_V, fmt, *V)
        bnd.attn_fwd_into(fmt, Q, K, V, shape, out, causal=causal, direct_p=direct_p, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        # eager work between replays: new inputs, written in place
        for x in (q, k, v):
            x.copy_(torch.randn(shape, generator=g, device="cuda").half())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_lse = out.clone(), lse.clone()
        out.fill_(float("nan")); lse.fill_(float("nan"))
        step()  # eager, same inputs
        torch.cuda.synchronize()
        say(f"  replay {r}: fmt={fmt} dp={direct_p} causal={causal}")
        assert torch.equal(got_out, out), f"replay {r}: output differs from eager"
        assert torch.equal(got_lse, lse), f"replay {r}: lse differs from eager"
        assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_graph_kv16_replays_match_eager(causal, fused):
    """The kv16 path captured as one graph: Q quantised, K and V either quantised and then
    dequantised by sage_fp4_kv16_prep or quantised by sage_fp4_quant_kv16 (fused), then
    sage_fp4_attn_fwd_kv16 with lse. Every replay, with new inputs written between replays, equals
    the eager run."""
    B, H, N, D = 2, 3, 500, 64
    shape = (B, H, N, D)
    fmt = bnd.NVFP4
    g = torch.Generator(device="cuda").manual_seed(13)
    q, k, v = (torch.randn(shape, generator=g, device="cuda").half() for _ in range(3))
    Q, K, V = (bnd.alloc_quant(r, fmt, *shape) for r in (bnd.ROLE_Q, bnd.ROLE_K, bnd.ROLE_V))
    kv = torch.empty(bnd.sage_fp4_kv16_bytes(*shape), dtype=torch.uint8, device="cuda")
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(B * H * N, dtype=torch.float32, device="cuda")

    def step():
        bnd.quant_into(q, bnd.ROLE_Q, fmt, *Q)
        if fused:
            bnd.quant_kv16_into(k, bnd.ROLE_K, *K, kv)
            bnd.quant_kv16_into(v, bnd.ROLE_V, *V, kv)
        else:
            bnd.quant_into(k, bnd.ROLE_K, fmt, *K)
            bnd.quant_into(v, bnd.ROLE_V, fmt, *V)
            bnd.kv16_prep(K, V, shape, kv)
        bnd.attn_fwd_kv16_into(Q, kv, shape, out, causal=causal, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for x in (q, k, v):
            x.copy_(torch.randn(shape, generator=g, device="cuda").half())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_lse = out.clone(), lse.clone()
        out.fill_(float("nan")); lse.fill_(float("nan")); kv.fill_(0x7B)
        step()
        torch.cuda.synchronize()
        say(f"  kv16 replay {r}: causal={causal} fused={fused}")
        assert torch.equal(got_out, out), f"replay {r}: output differs from eager"
        assert torch.equal(got_lse, lse), f"replay {r}: lse differs from eager"
        assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("fmt,causal", [(bnd.NVFP4, True), (bnd.MXFP4, False)])
def test_graph_training_step_replays_match_eager(fmt, causal):
    """Forward with the row log-sum-exp and the 8-bit backward (three quantisations, one
    attention launch, five backward launches) captured as one graph: every replay, with new
    inputs and output gradients written between replays, equals the eager run bit for bit."""
    B, H, N, D = 1, 4, 700, 128
    shape = (B, H, N, D)
    g = torch.Generator(device="cuda").manual_seed(12)
    q, k, v, do = (torch.randn(shape, generator=g, device="cuda").half() for _ in range(4))
    Q, K, V = (bnd.alloc_quant(r, fmt, *shape) for r in (bnd.ROLE_Q, bnd.ROLE_K, bnd.ROLE_V))
    out = torch.empty(shape, dtype=torch.float16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = [torch.empty(shape, dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)

    def step():
        bnd.quant_into(q, bnd.ROLE_Q, fmt, *Q)
        bnd.quant_into(k, bnd.ROLE_K, fmt, *K)
        bnd.quant_into(v, bnd.ROLE_V, fmt, *V)
        bnd.attn_fwd_into(fmt, Q, K, V, shape, out, causal=causal, lse=lse)
        bnd.attn_bwd_into(fmt, Q, K, v, out, do, lse, *grads, ws, causal=causal)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for x in (q, k, v, do):
            x.copy_(torch.randn(shape, generator=g, device="cuda").half())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in grads]
        for t in grads:
            t.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        say(f"  training-step replay {r}: fmt={fmt} causal={causal}")
        for a, b in zip(got, grads):
            assert torch.equal(a, b), f"replay {r}: gradients differ from eager"
            assert bool(torch.isfinite(b).all())
