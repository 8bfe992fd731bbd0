"""Benchmark of the FP4 microscaling attention forward on one MI355X.

One step = the whole hot path over one batch: sage_fp4_quant of Q, K and V, then
sage_fp4_attn_fwd, with the fp16 inputs already resident in HBM. Workload: B=4, H=32, N=4096,
D=128, NVFP4, non-causal (the kernel-sweep point), synthetic seeded inputs; --seq-len picks
another point of the N sweep at the same B, H, D (1024, 2048, 8192, 16384).

Prints one JSON line. `value` = 4*B*H*N^2*D / (step time) in TOPS (whole step, quantisation
included); the attention kernel alone is reported in `attn_*` fields and `roofline`, timed with
HIP events on the stream the kernels are launched on. `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.

`--sweep PATH` times the attention alone over the N sweep and workloads 3 and 4, every format and
mask, appending one JSON line per entry to PATH and skipping entries already there.

`--kv16` (NVFP4) makes the step quantise K and V with sage_fp4_quant_kv16, which also writes
their exact fp16 dequantisation in the same pass, and run sage_fp4_attn_fwd_kv16 on that buffer
(outputs identical to the default step's, bit for bit).

`--backward` times the 8-bit backward instead (sage_fp4_attn_bwd as its three stages, on the
forward's FP4 Q/K, output and log-sum-exp): `value` = 10*B*H*N^2*D / (backward time), the
roofline is that of its dK/dV kernel, and the CPU baseline is the backward oracle on one head.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 attention fwd TOPS (4·B·H·N²·D/t) + %FP4-MFMA peak; cos-sim vs FP32"
FP4_PEAK_TOPS = 10066.0      # MI355X dense FP4 MFMA (256 CU x 4 SIMD x 4096 flop/clk x 2.4 GHz)
FP8_PEAK_TOPS = 5033.0       # MI355X dense FP8 MFMA (half the FP4 rate)
FP16_PEAK_TFLOPS = 2516.6    # dense fp16 MFMA
HBM_PEAK_GBS = 8000.0
WORKLOAD = dict(B=4, H=32, N=4096, D=128)
WORKLOAD_NAMES = {2: "kernel sweep point", 3: "video-DiT shape", 4: "long-context causal"}
DATA_NOTES = {
    2: "synthetic (seeded SplitMix64/Box-Muller N(0,1) fp16)",
    3: "synthetic (seeded N(0,1) fp16; K plus per-(head, channel) offsets drawn N(0, sd 3))",
    4: "synthetic (seeded N(0,1) fp16; each entry +-20 with probability 0.001)"}
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(name: str) -> str:
    h = hashlib.sha256()
    for f in (name, "device.h"):
        with open(os.path.join(ROOT, "bit_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file: str, key: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(key)
    if not e or e.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    return e.get("bytes_per_launch")


def torch_reference_rows(q, k, v, heads, rows, sm_scale, causal=False):
    """Plain PyTorch fp32 attention on the GPU for a few (head, row) samples; with causal, key j
    is visible to query i iff j <= i."""
    import torch
    outs = []
    for h in heads:
        qh = q.view(-1, q.shape[2], q.shape[3])[h].float()
        kh = k.view(-1, k.shape[2], k.shape[3])[h].float().contiguous()
        vh = v.view(-1, v.shape[2], v.shape[3])[h].float().contiguous()
        s = torch.matmul(qh[rows], kh.t().contiguous()) * sm_scale
        if causal:
            keys = torch.arange(kh.shape[0], device=s.device)
            s = s.masked_fill(keys[None, :] > rows[:, None], float("-inf"))
        p = torch.softmax(s, dim=-1)
        outs.append(torch.matmul(p, vh))
    return torch.cat(outs).double().cpu().numpy()


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(q_np, k_np, v_np, shape, fmt, direct_p=False, seconds_target=15.0, gpu_out=None, gpu_qkv=None):
    """The oracle, as it stands, on a bounded sample of the same workload: head after head, the
    quantisation of the head's Q, K and V and the attention of every 4th query row of it, until
    about `seconds_target` seconds of CPU time; the quantisation is charged pro rata to the rows
    computed. Throughput by the same 4*N*D-per-row count as the GPU figure. If `gpu_out` (the
    non-causal GPU output, [B*H, N, D] on the host) is given, the largest |GPU - oracle| over the
    sampled rows is returned as well; if `gpu_qkv` (the GPU's Q, K, V codes and scales on the
    host, in the oracle's array shapes) is given, the number of code and scale bytes of the
    sampled heads that differ from the oracle's."""
    import oracle as orc
    B, H, N, D = shape
    nthreads = orc.max_threads()
    rows = np.arange(0, N, 4, dtype=np.int64)
    total_t, total_rows, heads = 0.0, 0, 0
    max_abs = 0.0
    mism = {"code_bytes_compared": 0, "code_bytes_differing": 0, "scale_bytes_compared": 0,
            "scale_bytes_differing": 0}
    for bh in range(B * H):
        b, h = divmod(bh, H)
        t0 = time.perf_counter()
        Q = orc.quant(orc.ROLE_Q, fmt, q_np[b:b + 1, h:h + 1])
        K = orc.quant(orc.ROLE_K, fmt, k_np[b:b + 1, h:h + 1])
        V = orc.quant(orc.ROLE_V, fmt, v_np[b:b + 1, h:h + 1])
        t_quant = time.perf_counter() - t0
        if gpu_qkv is not None:
            for (oc, os_), (gc, gs) in zip((Q, K, V), gpu_qkv):
                mism["code_bytes_compared"] += oc.size
                mism["code_bytes_differing"] += int(np.count_nonzero(oc[0, 0] != gc[b, h]))
                mism["scale_bytes_compared"] += os_.size
                mism["scale_bytes_differing"] += int(np.count_nonzero(os_[0, 0] != gs[b, h]))
        t0 = time.perf_counter()
        out = orc.attn_fwd(fmt, Q, K, V, (1, 1, N, D), rows=rows, nthreads=nthreads, direct_p=direct_p)
        t_attn = time.perf_counter() - t0
        assert np.all(np.isfinite(out))
        if gpu_out is not None:
            max_abs = max(max_abs, float(np.abs(gpu_out[bh][rows].astype(np.float64) - out).max()))
        total_t += t_attn + t_quant * len(rows) / N
        total_rows += len(rows)
        heads += 1
        if total_t >= seconds_target:
            break
    tops = 4.0 * N * D * total_rows / total_t / 1e12
    return {"value": tops, "unit": "TOPS", "cores": nthreads, "kind": "oracle", "cpu_model": cpu_model(),
            "quant_vs_oracle": mism if gpu_qkv is not None else None,
            "sample": f"{heads} heads x {len(rows)} query rows (every 4th row; non-causal, N={N}, "
                      f"D={D}), format {fmt}{' Direct-P' if direct_p else ''}: per head the quantisation of Q, K, V (charged "
                      f"{len(rows)}/{N}) and the attention rows; {total_t:.1f} s of CPU time",
            "seconds": total_t, "max_abs_gpu_vs_oracle": max_abs if gpu_out is not None else None}


def cpu_one_thread_small(fmt, direct_p=False):
    """The oracle on one thread over the whole small parity workload (B1 H2 N256 D64): quantisation
    of Q, K, V and every attention row."""
    import oracle as orc
    from bit_attention_amd import synth
    q, k, v = synth.make_qkv(1)
    B, H, N, D = q.shape
    t0 = time.perf_counter()
    Q = orc.quant(orc.ROLE_Q, fmt, q)
    K = orc.quant(orc.ROLE_K, fmt, k)
    V = orc.quant(orc.ROLE_V, fmt, v)
    orc.attn_fwd(fmt, Q, K, V, (B, H, N, D), nthreads=1, direct_p=direct_p)
    t = time.perf_counter() - t0
    return {"value": 4.0 * B * H * N * N * D / t / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"whole B{B} H{H} N{N} D{D} workload, non-causal (quantisation on the oracle's "
                      f"default threads), attention on 1 thread", "seconds": t}


def warm(fn, torch, min_seconds=0.15, max_calls=5000):
    """Run fn back to back until at least min_seconds have passed (and at least 3 calls): the
    GPU's clock ramps up over roughly the first 30 ms of sustained load, and an idle gap (host
    work between measurements) lets it fall again."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or (time.perf_counter() - t0 < min_seconds and n < max_calls):
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def copy_ceiling_gbs(torch):
    """Device-to-device copy of 1 GiB, timed with HIP events: bytes read + written per second."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del src, dst
    return 2.0 * (1 << 30) / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--causal", action="store_true", help="time the causal variant instead")
    ap.add_argument("--fmt", choices=["nvfp4", "mxfp4", "mx4_pv8"], default="nvfp4",
                    help="mx4_pv8: MXFP4 Q and K, MXFP8 P and V")
    ap.add_argument("--direct-p", action="store_true", help="time sage_fp4_attn_fwd_direct_p (mxfp4 only)")
    ap.add_argument("--kv16", action="store_true",
                    help="nvfp4: the step quantises K and V with sage_fp4_quant_kv16 (codes plus "
                         "their fp16 dequantisation) and runs sage_fp4_attn_fwd_kv16 on them")
    ap.add_argument("--seq-len", type=int, default=WORKLOAD["N"],
                    help="N of the sweep at B=4 H=32 D=128 (default 4096)")
    ap.add_argument("--workload", type=int, choices=[2, 3, 4], default=2,
                    help="3: video-DiT shape B1 H48 N17776 D64 with K channel offsets; 4: long causal "
                         "B1 H32 N32768 D128 with +-20 outliers (implies --causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the post-run extra measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the 8-bit backward instead (sage_fp4_attn_bwd, as its three stages)")
    ap.add_argument("--sweep", metavar="PATH",
                    help="time the attention alone over the N sweep (B4 H32 D128, N 1024..16384) and "
                         "workloads 3 and 4, every format and mask; one JSON line per entry appended "
                         "to PATH, entries already in PATH skipped (the sweep resumes)")
    ap.add_argument("--sweep-formats", default=",".join(f for f, _, _ in SWEEP_FORMATS),
                    help="comma-separated subset of the sweep's formats (default: all)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on exactly one GPU; multi-GPU runs are not supported "
              "(every (batch, head) is independent, so heads would shard with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_attention_amd import binding as bnd
    from bit_attention_amd import synth

    if args.sweep:
        fmts = [f for f in args.sweep_formats.split(",") if f]
        unknown = sorted(set(fmts) - {f for f, _, _ in SWEEP_FORMATS})
        if unknown:
            print(f"bench.py: unknown sweep formats {unknown}", file=sys.stderr)
            sys.exit(2)
        return run_sweep(args.sweep, torch, bnd, synth, fmts)
    fmt = {"nvfp4": bnd.NVFP4, "mxfp4": bnd.MXFP4, "mx4_pv8": bnd.MX4_PV8}[args.fmt]
    if args.direct_p and fmt != bnd.MXFP4:
        print("bench.py: --direct-p needs --fmt mxfp4", file=sys.stderr)
        sys.exit(2)
    if args.kv16 and (fmt != bnd.NVFP4 or args.backward):
        print("bench.py: --kv16 needs --fmt nvfp4 (forward)", file=sys.stderr)
        sys.exit(2)
    if args.workload == 2:
        B, H, D = (WORKLOAD[k] for k in "BHD")
        N = args.seq_len
        if N < 256 or N % 256:
            print("bench.py: --seq-len must be a positive multiple of 256", file=sys.stderr)
            sys.exit(2)
    else:
        w = synth.WORKLOADS[args.workload]
        B, H, N, D = w["B"], w["H"], w["N"], w["D"]
        args.causal = args.causal or w["causal"]
    shape = (B, H, N, D)
    if args.backward:
        return bench_backward(args, shape, fmt, torch, bnd, synth)
    log(f"bench: generating inputs {shape} ...")
    t0 = time.perf_counter()
    q_np, k_np, v_np = synth.make_qkv(2, N=N) if args.workload == 2 else synth.make_qkv(args.workload)
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    q = torch.from_numpy(q_np).to(dev)
    k = torch.from_numpy(k_np).to(dev)
    v = torch.from_numpy(v_np).to(dev)
    Q = bnd.alloc_quant(bnd.ROLE_Q, fmt, *shape)
    K = bnd.alloc_quant(bnd.ROLE_K, fmt, *shape)
    V = bnd.alloc_quant(bnd.ROLE_V, fmt, *shape)
    out = torch.empty(shape, dtype=torch.float16, device=dev)
    kv16 = torch.empty(bnd.sage_fp4_kv16_bytes(*shape), dtype=torch.uint8, device=dev) if args.kv16 else None
    stream = torch.cuda.current_stream()
    causal = args.causal

    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]

    def attention():
        if args.kv16:
            bnd.attn_fwd_kv16_into(Q, kv16, shape, out, causal=causal)
        else:
            bnd.attn_fwd_into(fmt, Q, K, V, shape, out, causal=causal, direct_p=args.direct_p)

    def step(i=None):
        if i is not None:
            ev[i][0].record(stream)
        bnd.quant_into(q, bnd.ROLE_Q, fmt, *Q)
        if args.kv16:
            bnd.quant_kv16_into(k, bnd.ROLE_K, *K, kv16)
            bnd.quant_kv16_into(v, bnd.ROLE_V, *V, kv16)
        else:
            bnd.quant_into(k, bnd.ROLE_K, fmt, *K)
            bnd.quant_into(v, bnd.ROLE_V, fmt, *V)
        if i is not None:
            ev[i][1].record(stream)
        attention()
        if i is not None:
            ev[i][2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))

    flops_formula = 4.0 * B * H * N * N * D
    flops = flops_formula / 2 if causal else flops_formula  # causal: masked work is skipped
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tops = flops / (attn_ms * 1e-3) / 1e12
    kfile = "attn_nvfp4.hip" if fmt == bnd.NVFP4 else "attn_mxfp4.hip"
    kname = {bnd.NVFP4: "attn_nvfp4", bnd.MXFP4: "attn_mxfp4", bnd.MX4_PV8: "attn_mx4pv8"}[fmt]
    kname += "_direct_p" if args.direct_p else ""
    kname += "_kv16" if args.kv16 else ""
    tkey = f"{kname}_b{B}_h{H}_n{N}_d{D}_{'causal' if causal else 'noncausal'}"
    traffic = load_traffic(kfile, tkey)
    # the metric's denominator is the dense FP4 MFMA peak for every format; the fraction of the
    # peak of the MFMA the kernel actually runs on is reported beside it
    if fmt == bnd.NVFP4 and args.kv16:
        own_peak = FP16_PEAK_TFLOPS
        kdesc = ("attn_nvfp4_kernel, KV16 instance (fp16 MFMA; K-hat and V-hat read dequantised, as the "
                 "K and V quantisers wrote them)")
    elif fmt == bnd.NVFP4:
        own_peak, kdesc = FP16_PEAK_TFLOPS, "attn_nvfp4_kernel (fp16 MFMA on exactly dequantised NVFP4 operands)"
    elif fmt == bnd.MXFP4:
        own_peak = FP4_PEAK_TOPS
        kdesc = "attn_mxfp4_kernel (block-scaled FP4 MFMA" + (", Direct-P normaliser)" if args.direct_p else ")")
    else:  # QK at the FP4 rate, PV at the FP8 rate
        own_peak = 2.0 / (1.0 / FP4_PEAK_TOPS + 1.0 / FP8_PEAK_TOPS)
        kdesc = "attn_mxfp4_kernel, FP8-PV instance (FP4 QK, FP8 PV MFMA)"
    roof = {"bound": "mfma", "achieved": attn_tops, "peak": FP4_PEAK_TOPS, "unit": "TFLOP/s",
            "frac": attn_tops / FP4_PEAK_TOPS, "traffic": traffic, "kernel": kdesc,
            "own_mfma_peak": own_peak, "frac_own_mfma_peak": attn_tops / own_peak}
    blk = 16 if fmt == bnd.NVFP4 else 32
    v_code_bytes = 1.0 if fmt == bnd.MX4_PV8 else 0.5  # MXFP8 V: one byte per element
    quant_bytes = B * H * N * D * (2 * (2 + 0.5 + 1.0 / blk) + (2 + v_code_bytes + 1.0 / blk))
    if args.kv16:  # K-hat and V-hat: 2 bytes per element of the padded rows
        quant_bytes += bnd.sage_fp4_kv16_bytes(*shape)
    res = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.fmt, "data": DATA_NOTES[args.workload],
        "config": {"workload": f"{WORKLOAD_NAMES[args.workload]} B={B} H={H} N={N} D={D} {args.fmt}"
                               f"{' direct-p' if args.direct_p else ''}{' kv16' if args.kv16 else ''}"
                               f" {'causal' if causal else 'non-causal'}",
                   "B": B, "H": H, "N": N, "D": D, "causal": causal, "format": args.fmt,
                   "kv_tile": bnd.sage_fp4_kv_tile(), "out_dtype": "f16"},
        "attn_kernel_ms": attn_ms, "attn_tops": attn_tops, "attn_frac_fp4_peak": attn_tops / FP4_PEAK_TOPS,
        "quant_ms_3_tensors": quant_ms, "quant_gbs": quant_bytes / (quant_ms * 1e-3) / 1e9,
        # not in counter runs: their one calibration copy must be the only copy kernel
        "copy_ceiling_gbs": None if args.calibrate_copy else copy_ceiling_gbs(torch),
        "flops_counted": flops, "flops_formula_4BHN2D": flops_formula,
        "roofline": roof,
    }

    # accuracy against a plain PyTorch fp32 reference on sampled rows of three heads
    torch.cuda.synchronize()
    heads = [0, B * H // 2 + 1, B * H - 1]
    rows = torch.arange(0, N, max(1, N // 256), device=dev)
    refs = {c: torch_reference_rows(q, k, v, heads, rows, 1.0 / np.sqrt(D), causal=c) for c in (False, True)}
    got = torch.cat([out.view(-1, N, D)[h][rows] for h in heads]).double().cpu().numpy()
    a, b = got.reshape(-1), refs[causal].reshape(-1)
    res["cos_sim_vs_fp32"] = float(a @ b / np.sqrt((a @ a) * (b @ b)))
    res["rel_l1_vs_fp32"] = float(np.abs(a - b).sum() / np.abs(b).sum())

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 256 << 20

    if not args.no_extras:
        # the same attention launch alone, back to back (warmed up for 0.15 s, then 10 timed
        # launches): the kernel-benchmark convention, without the quantisation kernels in between
        warm(attention, torch)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(10):
            attention()
        a1.record(stream)
        torch.cuda.synchronize()
        res["attn_alone_ms"] = a0.elapsed_time(a1) / 10
        res["attn_alone_tops"] = flops / (res["attn_alone_ms"] * 1e-3) / 1e12
        # the same step captured once as a HIP graph and replayed (no host launch gaps between
        # its four kernels); the library allocates, synchronises and memsets nothing
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        warm(graph.replay, torch)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(20):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = g0.elapsed_time(g1) / 20
        res["graph_value"] = flops / (res["graph_ms_per_step"] * 1e-3) / 1e12
        del graph
        extras = {}
        for name, f2, c2, dp in (("nvfp4_causal", bnd.NVFP4, True, False),
                                 ("mxfp4_noncausal", bnd.MXFP4, False, False),
                                 ("mxfp4_causal", bnd.MXFP4, True, False),
                                 ("mxfp4_direct_p_noncausal", bnd.MXFP4, False, True),
                                 ("mxfp4_direct_p_causal", bnd.MXFP4, True, True),
                                 ("mx4_pv8_noncausal", bnd.MX4_PV8, False, False),
                                 ("mx4_pv8_causal", bnd.MX4_PV8, True, False)):
            if f2 == fmt and c2 == causal and dp == args.direct_p:
                continue
            Q2 = bnd.quant(q, bnd.ROLE_Q, f2); K2 = bnd.quant(k, bnd.ROLE_K, f2); V2 = bnd.quant(v, bnd.ROLE_V, f2)
            warm(lambda: bnd.attn_fwd_into(f2, Q2, K2, V2, shape, out, causal=c2, direct_p=dp), torch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                bnd.attn_fwd_into(f2, Q2, K2, V2, shape, out, causal=c2, direct_p=dp)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            fl = flops_formula / 2 if c2 else flops_formula
            t = fl / (ms * 1e-3) / 1e12
            extras[name] = {"attn_kernel_ms": ms, "attn_tops": t, "frac_fp4_peak": t / FP4_PEAK_TOPS}
            # accuracy against the same fp32 reference rows (causal mask when causal)
            got = torch.cat([out.view(-1, N, D)[h][rows] for h in heads]).double().cpu().numpy()
            a, b = got.reshape(-1), refs[c2].reshape(-1)
            extras[name]["cos_sim_vs_fp32"] = float(a @ b / np.sqrt((a @ a) * (b @ b)))
            extras[name]["rel_l1_vs_fp32"] = float(np.abs(a - b).sum() / np.abs(b).sum())
            if f2 == bnd.MX4_PV8:  # half the flops at the FP4 rate (QK), half at the FP8 rate (PV)
                mixed = 2.0 / (1.0 / FP4_PEAK_TOPS + 1.0 / FP8_PEAK_TOPS)
                extras[name]["frac_fp4_fp8_mixed_peak"] = t / mixed
        if fmt == bnd.NVFP4 and not args.kv16:
            # the same NVFP4 operands through sage_fp4_kv16_prep + sage_fp4_attn_fwd_kv16 (outputs
            # equal bit for bit): the prep once, then the attention alone, both masks
            kv = torch.empty(bnd.sage_fp4_kv16_bytes(*shape), dtype=torch.uint8, device=dev)
            warm(lambda: bnd.kv16_prep(K, V, shape, kv), torch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                bnd.kv16_prep(K, V, shape, kv)
            e1.record(stream)
            torch.cuda.synchronize()
            prep = e0.elapsed_time(e1) / 10
            for c2 in (False, True):
                warm(lambda: bnd.attn_fwd_kv16_into(Q, kv, shape, out, causal=c2), torch)
                e0.record(stream)
                for _ in range(10):
                    bnd.attn_fwd_kv16_into(Q, kv, shape, out, causal=c2)
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 10
                t = (flops_formula / 2 if c2 else flops_formula) / (ms * 1e-3) / 1e12
                extras["nvfp4_kv16_" + ("causal" if c2 else "noncausal")] = {
                    "attn_kernel_ms": ms, "attn_tops": t, "frac_fp4_peak": t / FP4_PEAK_TOPS,
                    "kv16_prep_ms": prep, "prep_plus_attn_ms": prep + ms}
            # this step (same inputs and mask) with K and V quantised by sage_fp4_quant_kv16, which
            # also writes the fp16 buffer in the same pass, and the attention reading that buffer
            # (the --kv16 step); 10 steps back to back after warming up
            Kf = bnd.alloc_quant(bnd.ROLE_K, bnd.NVFP4, *shape)
            Vf = bnd.alloc_quant(bnd.ROLE_V, bnd.NVFP4, *shape)

            def kv_quant():
                bnd.quant_kv16_into(k, bnd.ROLE_K, *Kf, kv)
                bnd.quant_kv16_into(v, bnd.ROLE_V, *Vf, kv)

            def fused_step():
                bnd.quant_into(q, bnd.ROLE_Q, fmt, *Q)
                kv_quant()
                bnd.attn_fwd_kv16_into(Q, kv, shape, out, causal=causal)

            timed = {}
            for key, fn in (("ms_per_step", fused_step), ("kv_quant_ms", kv_quant)):
                warm(fn, torch)
                e0.record(stream)
                for _ in range(10):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                timed[key] = e0.elapsed_time(e1) / 10
            extras["nvfp4_kv16_step_" + ("causal" if causal else "noncausal")] = {
                **timed, "value": flops / (timed["ms_per_step"] * 1e-3) / 1e12}
            del kv, Kf, Vf
        res["extras"] = extras

    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample ...")
        ofmt = {bnd.NVFP4: 0, bnd.MXFP4: 1, bnd.MX4_PV8: 2}[fmt]
        gpu_out = None
        if not causal:  # the sample is non-causal; the GPU output of the last timed step
            bnd.attn_fwd_into(fmt, Q, K, V, shape, out, causal=False, direct_p=args.direct_p)
            torch.cuda.synchronize()
            gpu_out = out.view(B * H, N, D).float().cpu().numpy()
        # the GPU's codes and scales of the last step, in the oracle's array shapes
        Np = (N + 127) // 128 * 128
        vb = 128 if fmt == bnd.MX4_PV8 else 64
        gpu_qkv = [(Q[0].cpu().numpy().reshape(B, H, N, D // 2), Q[1].cpu().numpy().reshape(B, H, N, D // blk)),
                   (K[0].cpu().numpy().reshape(B, H, N, D // 2), K[1].cpu().numpy().reshape(B, H, N, D // blk)),
                   (V[0].cpu().numpy().reshape(B, H, Np // 128, D, vb), V[1].cpu().numpy().reshape(B, H, Np // 128, D, 128 // blk))]
        res["cpu_baseline"] = cpu_baseline(q_np, k_np, v_np, shape, ofmt, args.direct_p, gpu_out=gpu_out,
                                           gpu_qkv=gpu_qkv)
        # fp16 output: the GPU side is rounded once more (half an fp16 ulp, ~1e-3 at |o| ~ 2)
        res["max_abs_vs_oracle_f16_out"] = res["cpu_baseline"]["max_abs_gpu_vs_oracle"]
        res["cpu_one_thread_small_workload"] = cpu_one_thread_small(ofmt, args.direct_p)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


SWEEP_FORMATS = (("nvfp4", 0, False), ("nvfp4_kv16", 0, False), ("mxfp4", 1, False), ("mxfp4_direct_p", 1, True),
                 ("mx4_pv8", 2, False))


def run_sweep(path, torch, bnd, synth, formats):
    """The attention kernel alone (warmed up, 10 launches timed with HIP events on the launch
    stream) for every (shape, format, mask) entry; each entry is appended to `path` as one JSON
    line as soon as it is measured, and entries already in `path` are skipped. nvfp4_kv16 entries
    time sage_fp4_attn_fwd_kv16 and, apart, the sage_fp4_kv16_prep it reads."""
    done = set()
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line:
                    done.add(json.loads(line)["key"])
    shapes = [("N%d" % n, 2, (4, 32, n, 128), n) for n in (1024, 2048, 4096, 8192, 16384)]
    shapes += [("wl3", 3, None, None), ("wl4", 4, None, None)]
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda:0")
    for tag, wl, shape, n in shapes:
        if shape is None:
            w = synth.WORKLOADS[wl]
            shape = (w["B"], w["H"], w["N"], w["D"])
        masks = (True,) if wl == 4 else (False, True)
        todo = [(f, fv, dp, c) for f, fv, dp in SWEEP_FORMATS for c in masks
                if f in formats and f"{tag}_{f}_{'causal' if c else 'noncausal'}" not in done]
        if not todo:
            continue
        log(f"bench sweep: {tag} {shape}, {len(todo)} entries")
        q_np, k_np, v_np = synth.make_qkv(2, N=n) if wl == 2 else synth.make_qkv(wl)
        q, k, v = (torch.from_numpy(x).to(dev) for x in (q_np, k_np, v_np))
        del q_np, k_np, v_np
        out = torch.empty(shape, dtype=torch.float16, device=dev)
        B, H, N, D = shape
        for f, fv, dp, c in todo:
            Q, K, V = bnd.quant(q, bnd.ROLE_Q, fv), bnd.quant(k, bnd.ROLE_K, fv), bnd.quant(v, bnd.ROLE_V, fv)
            kv16 = prep_ms = None
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if f == "nvfp4_kv16":
                kv16 = torch.empty(bnd.sage_fp4_kv16_bytes(*shape), dtype=torch.uint8, device=dev)
                prep = lambda: bnd.kv16_prep(K, V, shape, kv16)  # noqa: E731
                warm(prep, torch)
                e0.record(stream)
                for _ in range(10):
                    prep()
                e1.record(stream)
                torch.cuda.synchronize()
                prep_ms = e0.elapsed_time(e1) / 10
                launch = lambda: bnd.attn_fwd_kv16_into(Q, kv16, shape, out, causal=c)  # noqa: E731
            else:
                launch = lambda: bnd.attn_fwd_into(fv, Q, K, V, shape, out, causal=c, direct_p=dp)  # noqa: E731
            warm(launch, torch)
            e0.record(stream)
            for _ in range(10):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            fl = 4.0 * B * H * N * N * D / (2 if c else 1)
            entry = {"key": f"{tag}_{f}_{'causal' if c else 'noncausal'}", "B": B, "H": H, "N": N, "D": D,
                     "format": f, "causal": c, "attn_kernel_ms": ms, "attn_tops": fl / (ms * 1e-3) / 1e12,
                     "frac_fp4_peak": fl / (ms * 1e-3) / 1e12 / FP4_PEAK_TOPS}
            if prep_ms is not None:
                entry["kv16_prep_ms"] = prep_ms
            with open(path, "a") as fh:
                fh.write(json.dumps(entry) + "\n")
            log(f"bench sweep: {entry['key']} {ms:.4f} ms {entry['attn_tops']:.0f} TOPS")
            del Q, K, V, kv16
        del q, k, v, out
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": path, "entries_skipped": len(done)}), flush=True)


BWD_METRIC = "8-bit attention bwd TOPS (10·B·H·N²·D/t: the five backward matmuls)"
INT8_PEAK_TOPS = 5033.0      # MI355X dense INT8 MFMA


def bench_backward(args, shape, fmt, torch, bnd, synth):
    """One step = sage_fp4_attn_bwd over the workload (its three stages, each bracketed by HIP
    events on the launch stream): operand preparation, dK/dV, dQ. Inputs resident in HBM: the
    forward's FP4 Q/K codes and its output and log-sum-exp (computed once, untimed), fp16 V and dO.
    Gradients are written in fp16."""
    B, H, N, D = shape
    causal = args.causal
    wl = args.workload
    log(f"bench: generating inputs {shape} ...")
    q_np, k_np, v_np = synth.make_qkv(2, N=N) if wl == 2 else synth.make_qkv(wl)
    do_np = synth.make_do(2, N=N) if wl == 2 else synth.make_do(wl)
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x).to(dev) for x in (q_np, k_np, v_np, do_np))
    Q = bnd.quant(q, bnd.ROLE_Q, fmt)
    K = bnd.quant(k, bnd.ROLE_K, fmt)
    V = bnd.quant(v, bnd.ROLE_V, fmt)
    o = torch.empty(shape, dtype=torch.float16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    bnd.attn_fwd_into(fmt, Q, K, V, shape, o, causal=causal, lse=lse)
    grads = [torch.empty(shape, dtype=torch.float16, device=dev) for _ in range(3)]
    ws = bnd.alloc_bwd_workspace(B, H, N, D)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(i=None):
        for s_, stage in enumerate((bnd.BWD_PREP, bnd.BWD_DKDV, bnd.BWD_DQ)):
            if i is not None:
                ev[i][s_].record(stream)
            bnd.attn_bwd_into(fmt, Q, K, v, o, do, lse, *grads, ws, causal=causal, stage=stage)
        if i is not None:
            ev[i][3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    st_ms = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) for j in range(3)]

    pairs = B * H * N * N / (2 if causal else 1)                 # visible (query, key) pairs, tile-level
    flops = 10.0 * B * H * N * N * D / (2 if causal else 1)      # five matmuls (S, dP, dV, dK, dQ), 2D each
    value = flops / (ms_step * 1e-3) / 1e12
    # the dK/dV kernel, per pair: S (2D flops; bf16 MFMA for NVFP4 Q/K, the block-scaled FP4 MFMA
    # for MXFP4 Q/K), dP at fp16 (2D) and dV, dK on INT8 (4D ops); the peak is the rate at which
    # that mix would run with every unit at its dense peak
    mx = args.fmt != "nvfp4"
    dkdv_ops = 8.0 * D * pairs
    dkdv_tops = dkdv_ops / (st_ms[1] * 1e-3) / 1e12
    s_peak = FP4_PEAK_TOPS if mx else FP16_PEAK_TFLOPS
    mixed = 8.0 / (2.0 / s_peak + 2.0 / FP16_PEAK_TFLOPS + 4.0 / INT8_PEAK_TOPS)
    kname = f"attn_bwd_dkdv_{'mxfp4_' if mx else ''}b{B}_h{H}_n{N}_d{D}_{'causal' if causal else 'noncausal'}"
    roof = {"bound": "mfma", "achieved": dkdv_tops, "peak": mixed, "unit": "TFLOP/s",
            "frac": dkdv_tops / mixed, "traffic": load_traffic("attn_bwd.hip", kname),
            "kernel": f"bwd_dkdv_kernel (S on the {'FP4' if mx else 'bf16'} MFMA, dP on fp16, dV and dK "
                      "on INT8; peak = the op-weighted harmonic mean of those dense peaks)"}
    res = {
        "metric": BWD_METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8+bf16/fp16", "data": DATA_NOTES[wl] + "; dO ~ N(0,1) fp16",
        "config": {"workload": f"backward, {WORKLOAD_NAMES[wl]} B={B} H={H} N={N} D={D} {args.fmt} Q/K "
                               f"{'causal' if causal else 'non-causal'}",
                   "B": B, "H": H, "N": N, "D": D, "causal": causal, "format": args.fmt, "grad_dtype": "f16"},
        "prep_ms": st_ms[0], "dkdv_ms": st_ms[1], "dq_ms": st_ms[2],
        "dq_tops": 6.0 * D * pairs / (st_ms[2] * 1e-3) / 1e12,
        "flops_counted": flops, "roofline": roof,
    }
    torch.cuda.synchronize()
    # accuracy: gradients of one head against float64 autograd (CPU) of unquantised attention
    h0 = B * H - 1

    def head(x):
        return torch.from_numpy(x.reshape(B * H, N, D)[h0].astype(np.float64))

    qh, kh, vh = (head(x).requires_grad_(True) for x in (q_np, k_np, v_np))
    doh = head(do_np)
    sc = (qh @ kh.T) / np.sqrt(D)
    if causal:
        sc = sc.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    (torch.softmax(sc, -1) @ vh * doh).sum().backward()
    for name, g, r in (("dq", grads[0], qh.grad), ("dk", grads[1], kh.grad), ("dv", grads[2], vh.grad)):
        a = g.view(B * H, N, D)[h0].double().cpu().numpy().reshape(-1)
        b = r.numpy().reshape(-1)
        res[f"cos_sim_{name}_vs_fp64"] = float(a @ b / np.sqrt((a @ a) * (b @ b)))
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 256 << 20
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_bwd(q_np, k_np, v_np, do_np, shape, fmt, causal)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def cpu_baseline_bwd(q_np, k_np, v_np, do_np, shape, fmt, causal, seconds_target=10.0):
    """The backward oracle (numpy, INT8 mode) on one head of the workload; its forward O and lse
    come from the oracle forward first (not timed)."""
    import oracle as orc
    from oracle import bwd as obwd
    B, H, N, D = shape
    h = B * H - 1
    qs, ks, vs, dos = (x.reshape(B * H, N, D)[h][None, None] for x in (q_np, k_np, v_np, do_np))
    fq = orc.MXFP4 if fmt == orc.MX4_PV8 else fmt
    Qs, Ks = orc.quant(0, fq, qs), orc.quant(1, fq, ks)
    o, lse = orc.attn_fwd(fmt, Qs, Ks, orc.quant(2, fmt, vs), qs.shape, causal=causal, want_lse=True)
    o16, l32 = o.astype(np.float16), lse.astype(np.float32).reshape(1, 1, N)
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or (time.perf_counter() - t0 < seconds_target and reps < 100):
        obwd.attn_bwd(fmt, Qs, Ks, vs, o16, dos, l32, causal=causal)
        reps += 1
    sec = time.perf_counter() - t0
    fl = reps * 10.0 * N * N * D / (2 if causal else 1)
    return {"value": fl / sec / 1e12, "unit": "TOPS", "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"one (batch, head) of the workload, N={N} D={D}, its backward run {reps} times in "
                      f"{sec:.1f} s (numpy float64 with BLAS threads; INT8 decisions in float32)"}


if __name__ == "__main__":
    main()
