#!/usr/bin/env python3
"""Throughput of the TQ4_1S dequantize-and-multiply path on one MI355X.

Headline (`value`): packed-weight GB/s of one dense denoiser-step projection,
M=16 tokens (one 16-token diffusion block), K=2688, N=8192, through
tq4_linear (activation rotation + dequant-GEMM).  A step is one such call;
the weights rotate over `--copies` distinct packed copies (48 x 13.76 MB =
660 MB, more than twice the 256 MB Infinity Cache), and the cache is flushed
before the timed steps, so every step streams its weights from HBM whatever
the step count.  Inputs are resident in HBM before timing starts.

Extra legs in the same JSON line: the M=4096 prefill projection (TFLOP/s,
Student-t weights) and the 128-expert top-6 MoE layer at 16 and 1024 tokens
(uniform and Zipf routing), each timed the same way, with its own roofline;
the offline quantizer's throughput; the fused bias + residual tail
(tq4_linear_epilogue) at M=16 and M=4096 against the plain call; and the fp8
weight-cache variant (tq4_fp8_cache / tq4_linear_fp8) on the same two shapes.

`roofline` is for the dominant kernel of the headline step: at M=16 the whole
tq4_linear call is one kernel (rotation fused), so its time per launch is the
step time.  Steps are launched back to back behind a spin on the GPU that
outlasts their submission (see time_loop), timed with HIP events on the
launch stream.  `cpu_baseline` times the fp64
CPU oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs all|none|a,b]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
LEAD_MIN_US = 1000.0           # GPU spin ahead of a timed region, at least this long
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
MFMA_F8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, TFLOP/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """The source without its comments and with runs of whitespace made one
    space, so that editing a comment leaves the hash of a kernel alone."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha(sources) -> str:
    """Hash of the code (comments and layout aside) of a kernel's sources."""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "block_diffusion_lm_tq4_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(key: str):
    """HBM bytes per launch from committed PMC counters, if they match the
    current source of the kernel they were taken on (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha(rec.get("sources", ())):
        return None
    return rec.get("hbm_bytes_per_launch")


_FLUSH = {}


def mall_flush(torch):
    """Read a 512 MiB buffer (twice the 256 MB Infinity Cache), so that no
    input of the next timed region is still cached from an earlier call.  A
    read leaves clean lines only: writing the buffer instead would leave
    dirty lines whose write-back would land inside the timed region."""
    from block_diffusion_lm_tq4_amd import ops
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
        _FLUSH["sink"] = torch.zeros(256, dtype=torch.float32, device="cuda")
        ops.read_probe(_FLUSH["buf"], _FLUSH["sink"])  # the zero fill's lines, written back
    ops.read_probe(_FLUSH["buf"], _FLUSH["sink"])


_SPIN = {}


def spin_cycles_per_us(torch) -> float:
    """Cycles of torch.cuda._sleep per microsecond on this GPU (measured once)."""
    if "rate" not in _SPIN:
        cycles = 4_000_000
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(10_000)
        s.record()
        torch.cuda._sleep(cycles)
        e.record()
        torch.cuda.synchronize()
        _SPIN["rate"] = cycles / (s.elapsed_time(e) * 1e3)
    return _SPIN["rate"]


def time_loop(torch, fn, steps: int, warmup: int) -> float:
    """Average ms per call of fn(i) over exactly `steps` calls.

    `warmup` calls first, then a device synchronization; a few more calls
    time the host's submission of one call.  A read of a 512 MiB buffer then
    evicts the Infinity Cache, so the timed calls read every input that they
    do not share from HBM, whatever the step count.  Behind it the GPU spins
    (torch.cuda._sleep) for four times the time the host needs to submit all
    `steps` calls plus 0.5 ms (at least 1 ms); the start event, the calls and the stop
    event are queued behind the spin on the launch stream (torch's current
    stream, which the library launches on), so when the spin ends every call
    is already queued and the GPU runs them back to back: the timed region
    holds the calls and neither the host's submission nor any launch work
    of its own.  A device synchronization ends it.  (Captured into a HIP
    graph and replayed instead, the same calls take the same time each, but
    each replay adds about 10 us before its first call: measured at M=16,
    17.0 us per call at 1 call per replay, 7.16 at 20, 6.68 at 100; queued
    eagerly behind the spin 9.6, 6.84 and 6.61.)  If the host's submission
    outlasted the spin the result would include its gaps, so that case is
    reported on stderr.
    """
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    n = max(1, min(steps, 8))
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    host_us = (time.perf_counter() - t0) * 1e6 / n
    torch.cuda.synchronize()
    lead_us = max(LEAD_MIN_US, 4.0 * steps * host_us + 500.0)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    cycles = int(lead_us * spin_cycles_per_us(torch))
    mall_flush(torch)
    torch.cuda._sleep(cycles)
    start.record()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    submit_us = (time.perf_counter() - t0) * 1e6
    stop.record()
    torch.cuda.synchronize()
    if submit_us > lead_us:
        print(f"[bench] warning: submitting {steps} calls took {submit_us:.0f} us, longer "
              f"than the {lead_us:.0f} us spin ahead of them", file=sys.stderr)
    return start.elapsed_time(stop) / steps


def time_graph_replay(torch, fn, steps: int, warmup: int) -> float:
    """time_loop's calls captured into a HIP graph and replayed instead of
    queued eagerly (same flush and spin ahead of the timed region); used by
    --timing-sweep to show what a replay adds per timed region."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    mall_flush(torch)
    torch.cuda._sleep(int(LEAD_MIN_US * spin_cycles_per_us(torch)))
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(stop) / steps


def timing_sweep(torch, np, ops, I, dev, sb, copies: int) -> dict:
    """Per-call time of the headline call against the number of calls in
    the timed region, eager behind the spin (time_loop) and graph-replayed
    (time_graph_replay): medians of five regions each."""
    wl = I.WORKLOADS["dense_m16"]
    packed = ops.pack(torch.from_numpy(I.weights(wl.n, wl.k, wl.weights)).to(dev), sb)
    stack = [packed] + [packed.clone() for _ in range(copies - 1)]
    x = bf16_dev(torch, np, I.activations_bf16(wl.m, wl.k), dev)
    y = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev)
    ws = torch.zeros(ops.linear_workspace_size(wl.m, wl.k, wl.n), dtype=torch.uint8, device=dev)

    def fn(i):
        ops.linear(x, stack[i % copies], sb, out=y, workspace=ws)

    out = {}
    for k in (1, 2, 5, 20, 100):
        e = sorted(time_loop(torch, fn, k, 5) * 1e3 for _ in range(5))
        g = sorted(time_graph_replay(torch, fn, k, 5) * 1e3 for _ in range(5))
        out[str(k)] = {"eager_us_per_call": round(e[2], 3), "graph_us_per_call": round(g[2], 3)}
        log("timing_sweep", f"K={k}: eager {e[2]:.3f} us per call, graph replay {g[2]:.3f}")
    return out


def bf16_dev(torch, np, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


# ----------------------------------------------------------------------------- legs

def dense_leg(torch, np, ops, I, wl, steps, warmup, copies, dev, sb):
    """Returns dict with step time, kernel time and work figures for a dense workload."""
    w = I.weights(wl.n, wl.k, wl.weights)
    packed = ops.pack(torch.from_numpy(w).to(dev), sb)
    del w
    stack = [packed] + [packed.clone() for _ in range(copies - 1)]
    x = bf16_dev(torch, np, I.activations_bf16(wl.m, wl.k), dev)
    y = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev)
    ws = torch.zeros(ops.linear_workspace_size(wl.m, wl.k, wl.n), dtype=torch.uint8, device=dev)
    xt = ops.act_rht(x, sb)

    def step(i):
        ops.linear(x, stack[i % copies], sb, out=y, workspace=ws)

    def kernel(i):
        ops.linear_rotated(xt, stack[i % copies], out=y, workspace=ws)

    ms_step = time_loop(torch, step, steps, warmup)
    # the dominant kernel alone: for m <= 16 the step is that one kernel
    ms_kernel = ms_step if wl.m <= 16 else time_loop(torch, kernel, steps, warmup)
    packed_bytes = packed.numel()
    flops = 2.0 * wl.m * wl.n * wl.k
    r = dict(ms_step=ms_step, ms_kernel=ms_kernel, packed_bytes=packed_bytes, flops=flops)
    if wl.m <= 16:
        # read ceiling: one plain streaming-read launch over the same packed
        # bytes, rotating over the same copies
        sink = torch.zeros(256, dtype=torch.float32, device=dev)
        r["ms_read"] = time_loop(torch, lambda i: ops.read_probe(stack[i % copies], sink),
                                 steps, warmup)
    else:
        # context: the vendor BLAS (torch.matmul -> hipBLASLt) on a dense fp16
        # GEMM of the same shape, fp16 out, weights already dense fp16
        a16 = xt.view(torch.float16)
        b16 = torch.randn((wl.n, wl.k), device=dev).to(torch.float16)
        c16 = torch.empty((wl.m, wl.n), dtype=torch.float16, device=dev)
        r["ms_dense_fp16_blas"] = time_loop(
            torch, lambda i: torch.matmul(a16, b16.t(), out=c16), steps, warmup)
        del b16, c16
    return r


def moe_setup(torch, np, ops, I, dev, sb, n1=1856, k=2688, n_exp=128):
    from concurrent.futures import ThreadPoolExecutor
    w1 = torch.empty((n_exp, n1, k // 32, 20), dtype=torch.uint8, device=dev)
    w2 = torch.empty((n_exp, k, n1 // 32, 20), dtype=torch.uint8, device=dev)

    def gen(e):
        return e, I.expert_weights(e, 1, n1, k), I.expert_weights(e, 2, n1, k)

    with ThreadPoolExecutor(8) as ex:
        for lo in range(0, n_exp, 16):
            for e, a, b in ex.map(gen, range(lo, min(lo + 16, n_exp))):
                w1[e] = ops.pack(torch.from_numpy(a).to(dev), sb)
                w2[e] = ops.pack(torch.from_numpy(b).to(dev), sb)
    return w1, w2


def moe_leg(torch, np, ops, I, wl, experts, steps, warmup, dev, sb, fp8=None):
    ids, g = I.moe_routing(wl)
    x = bf16_dev(torch, np, I.activations_bf16(wl.t, wl.k), dev)
    idt = torch.from_numpy(ids).to(dev)
    gt = torch.from_numpy(g).to(dev)
    out = torch.empty((wl.t, wl.k), dtype=torch.float32, device=dev)
    ws = torch.zeros(ops.moe_workspace_size(wl.t, wl.topk, wl.n_experts, wl.n1, wl.k),
                     dtype=torch.uint8, device=dev)

    def step(i):
        ops.moe_grouped(x, idt, gt, experts[0], experts[1], sb, out=out, workspace=ws)

    ms = time_loop(torch, step, steps, warmup)
    # the router in front of the layer (softmax + top-k on the device), on the
    # logits these ids came from
    lg = torch.from_numpy(I.router_logits(wl.t, wl.n_experts, wl.routing).astype(np.float32)).to(dev)
    r_ids = torch.empty_like(idt)
    r_g = torch.empty_like(gt)
    ms_router = time_loop(torch, lambda i: ops.moe_router(lg, wl.topk, r_ids, r_g), steps, warmup)
    # the whole block from the same logits in one call (tq4_moe_block)
    wsb = torch.zeros(ops.moe_block_workspace_size(wl.t, wl.topk, wl.n_experts, wl.n1, wl.k),
                      dtype=torch.uint8, device=dev)
    ms_block = time_loop(torch, lambda i: ops.moe_block(x, lg, wl.topk, experts[0], experts[1], sb,
                                                        out=out, workspace=wsb), steps, warmup)
    # the same block as one persistent launch (tq4_moe_block_persistent), where
    # its 16-row tiles apply
    ms_persistent = None
    wsp_bytes = ops.moe_block_persistent_workspace_size(wl.t, wl.topk, wl.n_experts, wl.n1, wl.k)
    if wsp_bytes > 0:
        wsp = torch.zeros(wsp_bytes, dtype=torch.uint8, device=dev)
        ms_persistent = time_loop(torch, lambda i: ops.moe_block_persistent(
            x, lg, wl.topk, experts[0], experts[1], sb, out=out, workspace=wsp), steps, warmup)
    touched = np.unique(ids).size
    per_expert = (wl.n1 * (wl.k // 32) + wl.k * (wl.n1 // 32)) * 20
    pairs = wl.t * wl.topk
    r = dict(ms_step=ms, ms_router=ms_router, ms_block=ms_block, ms_persistent=ms_persistent,
             packed_bytes=touched * per_expert,
             flops=2.0 * pairs * 2 * wl.n1 * wl.k, experts_touched=int(touched))
    if fp8 is not None:
        # the same layer on resident fp8 copies of the experts (tq4_moe_grouped_fp8)
        ws8 = torch.zeros(ops.moe_grouped_fp8_workspace_size(wl.t, wl.topk, wl.n_experts, wl.n1,
                                                             wl.k), dtype=torch.uint8, device=dev)
        out8 = torch.empty_like(out)
        r["ms_fp8"] = time_loop(torch, lambda i: ops.moe_grouped_fp8(
            x, idt, gt, fp8[0], fp8[1], wl.n_experts, wl.n1, out=out8, workspace=ws8),
            steps, warmup)
        kp, n1p = (wl.k + 127) // 128 * 128, (wl.n1 + 127) // 128 * 128
        r["fp8_bytes"] = touched * (wl.n1 * kp + wl.k * n1p) * 33 // 32
    return r


def epilogue_leg(torch, np, ops, I, wl, steps, warmup, copies, dev, sb):
    """The fused bias + residual tail (tq4_linear_epilogue, the residual being
    the output itself, as in a residual stream) against the same call without
    a tail and against that call followed by the two adds as torch kernels;
    and the bf16 residual stream form (tq4_linear_epilogue_bf16)."""
    w = I.weights(wl.n, wl.k, wl.weights)
    packed = ops.pack(torch.from_numpy(w).to(dev), sb)
    del w
    stack = [packed] + [packed.clone() for _ in range(copies - 1)]
    x = bf16_dev(torch, np, I.activations_bf16(wl.m, wl.k), dev)
    y = torch.zeros((wl.m, wl.n), dtype=torch.float32, device=dev)
    t = torch.empty_like(y)
    bias = torch.randn(wl.n, dtype=torch.float32, device=dev)
    ws = torch.zeros(ops.linear_workspace_size(wl.m, wl.k, wl.n), dtype=torch.uint8, device=dev)

    def fused(i):
        ops.linear_epilogue(x, stack[i % copies], sb, bias=bias, residual=y, out=y, workspace=ws)

    def plain(i):
        ops.linear(x, stack[i % copies], sb, out=t, workspace=ws)

    def unfused(i):
        plain(i)
        t.add_(bias)
        y.add_(t)

    y16 = torch.zeros((wl.m, wl.n), dtype=torch.bfloat16, device=dev)

    def fused_bf16(i):
        ops.linear_epilogue_bf16(x, stack[i % copies], sb, bias=bias, residual=y16, out=y16,
                                 workspace=ws)

    ms_f = time_loop(torch, fused, steps, warmup)
    ms_p = time_loop(torch, plain, steps, warmup)
    ms_u = time_loop(torch, unfused, steps, warmup)
    ms_h = time_loop(torch, fused_bf16, steps, warmup)
    return {"shape": f"{wl.m}x{wl.k}x{wl.n}", "fused_us": round(ms_f * 1e3, 2),
            "no_tail_us": round(ms_p * 1e3, 2), "linear_then_torch_adds_us": round(ms_u * 1e3, 2),
            "tail_cost_us": round((ms_f - ms_p) * 1e3, 2),
            "tail_bytes": wl.m * wl.n * 4 + wl.n * 4,
            "fused_bf16_stream_us": round(ms_h * 1e3, 2)}


def fp8_leg(torch, np, ops, I, wl, steps, warmup, copies, dev, sb):
    """The fp8 weight-cache variant on one dense workload: the one-time cache
    build, a step (activation quantization + product, tq4_linear_fp8) and the
    product alone (tq4_linear_fp8_quantized), the cache rotating over
    `copies` distinct copies."""
    w = I.weights(wl.n, wl.k, wl.weights)
    packed = ops.pack(torch.from_numpy(w).to(dev), sb)
    del w
    cache = ops.fp8_cache(packed, sb)
    ms_build = time_loop(torch, lambda i: ops.fp8_cache(packed, sb, out=cache), 5, 1)
    stack = [cache] + [cache.clone() for _ in range(copies - 1)]
    x = bf16_dev(torch, np, I.activations_bf16(wl.m, wl.k), dev)
    y = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(ops.linear_fp8_workspace_size(wl.m, wl.k, wl.n), 256),
                     dtype=torch.uint8, device=dev)
    codes, scales = ops.act_mxfp8(x)
    ms_step = time_loop(torch, lambda i: ops.linear_fp8(x, stack[i % copies], wl.n, out=y,
                                                        workspace=ws), steps, warmup)
    ms_kernel = time_loop(torch, lambda i: ops.linear_fp8_quantized(
        codes, scales, wl.k, stack[i % copies], wl.n, out=y), steps, warmup)
    r = dict(ms_build=ms_build, ms_step=ms_step, ms_kernel=ms_kernel, cache_bytes=cache.numel(),
             flops=2.0 * wl.m * wl.n * wl.k)
    if wl.m > 16:
        # context: the vendor BLAS fp8 GEMM (torch._scaled_mm -> hipBLASLt), e4m3 operands
        # with per-tensor scales, fp32 out, same shape
        try:
            a8 = torch.randn((wl.m, wl.k), device=dev).to(torch.float8_e4m3fn)
            b8 = torch.randn((wl.n, wl.k), device=dev).to(torch.float8_e4m3fn)
            one = torch.ones((), device=dev)
            c32 = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev)
            torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.float32)
            r["ms_fp8_blas"] = time_loop(torch, lambda i: torch._scaled_mm(
                a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.float32, out=c32),
                steps, warmup)
        except Exception as e:  # the library path is optional context
            r["fp8_blas_error"] = f"{type(e).__name__}: {str(e)[:120]}"
    return r


def rotation_ab_leg(torch, np, ops, I, steps, warmup, copies, dev, sb):
    """The rotation placement and the product arithmetic, measured
    (tq4_linear_variant): at M=16 the library's product (activation rotation,
    MFMA), the rotation undone on the weight tiles (MFMA products), and the
    products on the VALU; at M=4096 the two placements."""
    out = {}
    for name, variants, cps, st, wu in (
            ("dense_m16", ("default", "weight_rotation", "valu_product"), copies, steps, warmup),
            ("dense_m4096_t3", ("default", "weight_rotation"), 2, max(5, steps // 20),
             max(2, warmup // 10))):
        wl = I.WORKLOADS[name]
        w = I.weights(wl.n, wl.k, wl.weights)
        packed = ops.pack(torch.from_numpy(w).to(dev), sb)
        del w
        stack = [packed] + [packed.clone() for _ in range(cps - 1)]
        x = bf16_dev(torch, np, I.activations_bf16(wl.m, wl.k), dev)
        y = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(ops.linear_workspace_size(wl.m, wl.k, wl.n), wl.m * wl.k * 2),
                         dtype=torch.uint8, device=dev)
        leg = {}
        for v in variants:
            ms = time_loop(torch, lambda i, v=v: ops.linear_variant(
                x, stack[i % cps], sb, v, out=y, workspace=ws), st, wu)
            leg[v] = {"us": round(ms * 1e3, 2)}
            if wl.m <= 16:
                leg[v]["GB/s"] = round(packed.numel() / (ms * 1e-3) / 1e9, 1)
            else:
                leg[v]["TFLOP/s"] = round(2.0 * wl.m * wl.n * wl.k / (ms * 1e-3) / 1e12, 1)
        out[name] = leg
        del stack, packed
    return out


def pack_leg(torch, np, ops, I, steps, warmup, dev, sb, n=8192, k=2688):
    """Offline quantizer throughput (tq4_pack_bf16 and tq4_pack) on one
    denoiser-projection-sized matrix, weights resident on the device."""
    w = I.weights(n, k)
    w32 = torch.from_numpy(w).to(dev)
    wbf = w32.to(torch.bfloat16)
    out = torch.empty((n, k // 32, 20), dtype=torch.uint8, device=dev)
    ms_bf = time_loop(torch, lambda i: ops.pack(wbf, sb, out=out), steps, warmup)
    ms_32 = time_loop(torch, lambda i: ops.pack(w32, sb, out=out), steps, warmup)
    wps = n * k / (ms_bf * 1e-3)
    return {"matrix": f"{n}x{k}", "bf16_in_us": round(ms_bf * 1e3, 2),
            "fp32_in_us": round(ms_32 * 1e3, 2),
            "bf16_in_GB/s": round(n * k * 2 / (ms_bf * 1e-3) / 1e9, 1),
            "weights_per_s": float(f"{wps:.4g}"),
            "context": "59e9 weights (both towers) at this rate take "
                       f"{59e9 / wps:.1f} s of kernel time"}


# ----------------------------------------------------------------------- CPU side

CPU_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def cpu_host():
    """CPU model, logical CPU count and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def cpu_units(budget_s: float):
    """The fp64 oracle on bounded samples of each workload's unit of work,
    each sample repeated for about budget_s seconds in this process.  Returns
    {unit: {"work": amount per second, "unit", "calls", "seconds", "sample"}}."""
    import numpy as np

    import oracle as O
    from block_diffusion_lm_tq4_amd import inputs as I

    sb = I.sign_bits()
    units = {}

    def timed(name, fn, work, unit, sample):
        fn()  # first call outside the clock (page faults, BLAS start-up)
        calls, t0 = 0, time.perf_counter()
        while True:
            fn()
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        units[name] = {"work": work * calls / el, "unit": unit, "calls": calls,
                       "seconds": round(el, 2), "sample": sample}

    # dense M=16: 1024 of the 8192 weight rows; unit = packed bytes
    p16 = O.pack(I.weights(1024, 2688), sb)
    x16 = I.activations_bf16(16, 2688)
    timed("dense_m16", lambda: O.linear(x16, p16, sb), p16.nbytes, "B/s",
          "M=16, K=2688, 1024 of 8192 weight rows: unpack + rotate + fp64 matmul")
    # dense M=4096 (Student-t weights): all 4096 tokens against 64 weight rows
    p4k = O.pack(I.weights(64, 2688, "student_t3"), sb)
    x4k = I.activations_bf16(4096, 2688)
    timed("dense_m4096_t3", lambda: O.linear(x4k, p4k, sb), 2.0 * 4096 * 64 * 2688, "FLOP/s",
          "M=4096, K=2688, 64 of 8192 weight rows")
    # MoE, 16 tokens: the layer restricted to one expert that every token
    # routes to (top-1, gate 1); unit = that expert's packed bytes
    e_up = O.pack(I.expert_weights(0, 1), sb)
    e_dn = O.pack(I.expert_weights(0, 2), sb)
    xm = I.activations_bf16(16, 2688)
    ids = np.zeros((16, 1), dtype=np.int32)
    g = np.ones((16, 1), dtype=np.float32)
    timed("moe_t16", lambda: O.moe(xm, ids, g, [e_up], [e_dn], sb),
          e_up.nbytes + e_dn.nbytes, "B/s",
          "16 tokens through one 1856x2688 / 2688x1856 expert (both projections)")
    # the encoder: 256 rows of the dense projection; unit = weights
    wp = I.weights(256, 2688)
    timed("pack", lambda: O.pack(wp, sb), wp.size, "weights/s", "256 x 2688 fp32 weights")
    return units


def _cpu_worker(budget_s):
    return cpu_units(budget_s)


def cpu_leg_main(kind: str, workers: int, budget_s: float) -> int:
    """Entry of the child process that times the oracle (no GPU use here)."""
    if kind == "single":
        res = cpu_units(budget_s)
    else:
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(workers) as ex:
            parts = list(ex.map(_cpu_worker, [budget_s] * workers))
        res = {}
        for name in parts[0]:
            res[name] = dict(parts[0][name])
            res[name]["work"] = sum(p[name]["work"] for p in parts)
            res[name]["calls"] = sum(p[name]["calls"] for p in parts)
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline(budget_s: float = 2.5):
    """The fp64 oracle timed on this host, single-threaded and on all cores.

    Each leg runs in a child process that never touches the GPU, with the
    BLAS thread count fixed through the environment: single-threaded (one
    process, one BLAS thread) and all-core (one single-threaded process per
    available CPU, up to 16, each running the same samples; the samples are
    independent row or expert slices, so their rates add)."""
    import subprocess
    host = cpu_host()
    workers = max(1, min(host["affinity"], 16))
    legs = {}
    for kind, n in (("single", 1), ("all", workers)):
        env = dict(os.environ)
        for v in CPU_BLAS_ENV:
            env[v] = "1"
        cmd = [sys.executable, os.path.abspath(__file__), "--cpu-leg", kind,
               "--cpu-workers", str(n), "--cpu-budget", str(budget_s)]
        res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600)
        if res.returncode != 0:
            raise RuntimeError(f"cpu leg {kind} failed: {res.stderr[-2000:]}")
        legs[kind] = json.loads(res.stdout.strip().splitlines()[-1])

    def fmt(u):
        scale = {"B/s": (1e-9, "GB/s"), "FLOP/s": (1e-9, "GFLOP/s"),
                 "weights/s": (1e-6, "Mweights/s")}[u["unit"]]
        return {"value": float(f"{u['work'] * scale[0]:.4g}"), "unit": scale[1],
                "calls": u["calls"], "seconds": u["seconds"], "sample": u["sample"]}

    single = {k: fmt(v) for k, v in legs["single"].items()}
    allc = {k: fmt(v) for k, v in legs["all"].items()}
    return {"value": allc["dense_m16"]["value"], "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": "dense M=16 K=2688 projection, 1024 of 8192 weight rows (unpack + "
                      f"rotate + fp64 matmul), {workers} single-threaded processes",
            "host": host, "single_thread": single, "all_core": allc}


# ---------------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=48)
    ap.add_argument("--legs", default="all",
                    help="all | none | comma list of linear_512x256,dense_m4096_t3,moe_t16,"
                         "rotation_ab,"
                         "moe_t1024_uniform,moe_t1024_zipf,pack,epilogue,fp8")
    ap.add_argument("--only", default=None,
                    help="profile helper: run just this workload (no JSON contract)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timing-sweep", action="store_true",
                    help="print the headline call's per-call time against the calls per timed "
                         "region, eager and graph-replayed (no JSON contract)")
    ap.add_argument("--cpu-leg", choices=("single", "all"), default=None,
                    help=argparse.SUPPRESS)
    ap.add_argument("--cpu-workers", type=int, default=1, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-budget", type=float, default=2.5, help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --only: also run a plain 512 MiB device copy three times, "
                         "the reference for scaling HBM byte counters")
    args = ap.parse_args()

    if args.cpu_leg:
        return cpu_leg_main(args.cpu_leg, args.cpu_workers, args.cpu_budget)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from block_diffusion_lm_tq4_amd import inputs as I
    from block_diffusion_lm_tq4_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    sb = I.sign_bits()

    if args.timing_sweep:
        print(json.dumps({"timing_sweep": timing_sweep(torch, np, ops, I, dev, sb, args.copies)}))
        return 0
    if args.only:
        if args.only == "rotation_ab":
            r = rotation_ab_leg(torch, np, ops, I, args.steps, args.warmup, args.copies, dev, sb)
            log(args.only, json.dumps(r))
            return 0
        if args.only.startswith("fp8_"):
            wl = I.WORKLOADS[args.only[4:]]
            r = fp8_leg(torch, np, ops, I, wl, args.steps, args.warmup,
                        24 if wl.m <= 16 else 2, dev, sb)
            log(args.only, json.dumps(r))
            return 0
        wl = I.WORKLOADS[args.only]
        if args.only.startswith("dense"):
            r = dense_leg(torch, np, ops, I, wl, args.steps, args.warmup, args.copies, dev, sb)
        else:
            ex = moe_setup(torch, np, ops, I, dev, sb)
            ex8 = (ops.fp8_cache_experts(ex[0], sb), ops.fp8_cache_experts(ex[1], sb))
            r = moe_leg(torch, np, ops, I, wl, ex, args.steps, args.warmup, dev, sb, fp8=ex8)
        log(args.only, json.dumps(r))
        if args.copy_calibration:
            src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            log("copy calibration: 3 x 536870912 bytes read and written")
        return 0

    wl = I.WORKLOADS["dense_m16"]
    log("dense_m16: packing weights")
    r = dense_leg(torch, np, ops, I, wl, args.steps, args.warmup, args.copies, dev, sb)
    gbs = r["packed_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    k_gbs = r["packed_bytes"] / (r["ms_kernel"] * 1e-3) / 1e9
    read_gbs = r["packed_bytes"] / (r["ms_read"] * 1e-3) / 1e9
    log(f"dense_m16: step {r['ms_step'] * 1e3:.2f} us ({gbs:.0f} GB/s), "
        f"dequant-GEMM kernel {r['ms_kernel'] * 1e3:.2f} us ({k_gbs:.0f} GB/s), "
        f"plain read of the same bytes {r['ms_read'] * 1e3:.2f} us ({read_gbs:.0f} GB/s)")
    roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                "traffic": load_traffic("dense_m16"),
                "kernel": "skinny_dma_kernel (the whole tq4_linear call), algorithmic bytes per "
                          f"launch = packed weights {r['packed_bytes']}",
                "measured_ceiling": {"what": "one streaming-read launch (tq4_read_probe) over "
                                             "the same packed bytes and copies",
                                     "GB/s": round(read_gbs, 1),
                                     "frac_of_ceiling": round(k_gbs / read_gbs, 4)}}

    legs = {}
    names = ([] if args.legs == "none" else
             ["linear_512x256", "dense_m4096_t3", "moe_t16", "moe_t1024_uniform",
              "moe_t1024_zipf", "pack", "epilogue", "fp8", "rotation_ab"]
             if args.legs == "all" else args.legs.split(","))
    experts = fp8_experts = None
    for name in names:
        if name == "pack":
            log("pack: running")
            legs[name] = pack_leg(torch, np, ops, I, max(5, args.steps // 20), 2, dev, sb)
            log(name, json.dumps(legs[name]))
            continue
        if name == "fp8":
            log("fp8: running")
            q16 = fp8_leg(torch, np, ops, I, I.WORKLOADS["dense_m16"], max(5, args.steps // 2),
                          max(2, args.warmup // 2), 24, dev, sb)
            q4k = fp8_leg(torch, np, ops, I, I.WORKLOADS["dense_m4096_t3"],
                          max(5, args.steps // 20), max(2, args.warmup // 10), 2, dev, sb)
            k16 = q16["cache_bytes"] / (q16["ms_kernel"] * 1e-3) / 1e9
            t4k = q4k["flops"] / (q4k["ms_kernel"] * 1e-3) / 1e12
            leg = {
                "dense_m16": {
                    "step_us": round(q16["ms_step"] * 1e3, 2),
                    "product_us": round(q16["ms_kernel"] * 1e3, 2),
                    "tq4_step_us": round(r["ms_step"] * 1e3, 2),
                    "cache_bytes": q16["cache_bytes"],
                    "cache_build_us": round(q16["ms_build"] * 1e3, 1),
                    "roofline": {"bound": "hbm", "achieved": round(k16, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(k16 / HBM_PEAK_GBS, 4),
                                 "kernel": "fp8_stream_kernel (tq4_linear_fp8_quantized), "
                                           "algorithmic bytes = fp8 cache (codes + scales)"}},
                "dense_m4096_t3": {
                    "step_ms": round(q4k["ms_step"], 4),
                    "product_ms": round(q4k["ms_kernel"], 4),
                    "TFLOP/s": round(t4k, 1),
                    "roofline": {"bound": "mfma", "achieved": round(t4k, 1),
                                 "peak": MFMA_F8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(t4k / MFMA_F8_PEAK_TFLOPS, 4),
                                 "kernel": "fp8_gemm_kernel (tq4_linear_fp8_quantized), "
                                           "2*M*N*K flops per launch"}}}
            if "ms_fp8_blas" in q4k:
                bt = q4k["flops"] / (q4k["ms_fp8_blas"] * 1e-3) / 1e12
                leg["dense_m4096_t3"]["context_fp8_blas"] = {
                    "what": "torch._scaled_mm (hipBLASLt) e4m3 x e4m3 -> fp32, per-tensor "
                            "scales, same shape",
                    "TFLOP/s": round(bt, 1), "ours_over_blas": round(t4k / bt, 4)}
            elif "fp8_blas_error" in q4k:
                leg["dense_m4096_t3"]["context_fp8_blas"] = {"error": q4k["fp8_blas_error"]}
            legs[name] = leg
            log(name, json.dumps(leg))
            continue
        if name == "rotation_ab":
            log("rotation_ab: running")
            legs[name] = rotation_ab_leg(torch, np, ops, I, max(5, args.steps // 2),
                                         max(2, args.warmup // 2), args.copies, dev, sb)
            log(name, json.dumps(legs[name]))
            continue
        if name == "epilogue":
            log("epilogue: running")
            legs[name] = {
                "dense_m16": epilogue_leg(torch, np, ops, I, I.WORKLOADS["dense_m16"],
                                          max(5, args.steps // 2), max(2, args.warmup // 2),
                                          args.copies, dev, sb),
                "dense_m4096_t3": epilogue_leg(torch, np, ops, I, I.WORKLOADS["dense_m4096_t3"],
                                               max(5, args.steps // 20),
                                               max(2, args.warmup // 10), 2, dev, sb)}
            log(name, json.dumps(legs[name]))
            continue
        wl2 = I.WORKLOADS[name]
        if name == "linear_512x256":
            # the small parity layer: latency-bound, reported in microseconds
            log(f"{name}: running")
            q = dense_leg(torch, np, ops, I, wl2, max(5, args.steps // 2),
                          max(2, args.warmup // 2), args.copies, dev, sb)
            legs[name] = {"us_per_call": round(q["ms_step"] * 1e3, 3),
                          "plain_read_us": round(q["ms_read"] * 1e3, 3),
                          "packed_bytes": q["packed_bytes"],
                          "shape": f"M={wl2.m} K={wl2.k} N={wl2.n}",
                          "note": "no roofline target: 81,920 packed bytes per call"}
            log(name, json.dumps(legs[name]))
            continue
        if name.startswith("dense"):
            log(f"{name}: running")
            s2 = max(5, args.steps // 20)
            q = dense_leg(torch, np, ops, I, wl2, s2, max(2, args.warmup // 10), 2, dev, sb)
            tf = q["flops"] / (q["ms_step"] * 1e-3) / 1e12
            ktf = q["flops"] / (q["ms_kernel"] * 1e-3) / 1e12
            btf = q["flops"] / (q["ms_dense_fp16_blas"] * 1e-3) / 1e12
            legs[name] = {"ms_per_step": round(q["ms_step"], 4), "TFLOP/s": round(tf, 1),
                          "kernel_ms": round(q["ms_kernel"], 4),
                          "roofline": {"bound": "mfma", "achieved": round(ktf, 1),
                                       "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(ktf / MFMA_F16_PEAK_TFLOPS, 4),
                                       "traffic": load_traffic(name),
                                       "kernel": "gemm_huge_kernel (tq4_linear_rotated), "
                                                 "2*M*N*K flops per launch"},
                          "context_dense_fp16_blas": {
                              "what": "torch.matmul (hipBLASLt) fp16 x fp16 -> fp16 on the same "
                                      "shape, weights dense",
                              "TFLOP/s": round(btf, 1),
                              "ours_over_blas": round(ktf / btf, 4)}}
        else:
            if experts is None:
                log("moe: generating and packing 128 experts")
                experts = moe_setup(torch, np, ops, I, dev, sb)
                fp8_experts = (ops.fp8_cache_experts(experts[0], sb),
                               ops.fp8_cache_experts(experts[1], sb))
            log(f"{name}: running")
            s2 = max(5, args.steps // 10)
            q = moe_leg(torch, np, ops, I, wl2, experts, s2, max(2, args.warmup // 5), dev, sb,
                        fp8=fp8_experts)
            g2 = q["packed_bytes"] / (q["ms_step"] * 1e-3) / 1e9
            tf = q["flops"] / (q["ms_step"] * 1e-3) / 1e12
            legs[name] = {"ms_per_step": round(q["ms_step"], 4), "GB/s": round(g2, 1),
                          "TFLOP/s": round(tf, 2), "experts_touched": q["experts_touched"],
                          "router_us": round(q["ms_router"] * 1e3, 2),
                          "block_from_logits_us": round(q["ms_block"] * 1e3, 2),
                          "block_persistent_us": (None if q["ms_persistent"] is None else
                                                  round(q["ms_persistent"] * 1e3, 2)),
                          "roofline": {"bound": "hbm", "achieved": round(g2, 1),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(g2 / HBM_PEAK_GBS, 4)},
                          "fp8_cache": {
                              "what": "the same layer on resident MXFP8 expert copies "
                                      "(tq4_moe_grouped_fp8), GB/s on their touched bytes",
                              "ms_per_step": round(q["ms_fp8"], 4),
                              "GB/s": round(q["fp8_bytes"] / (q["ms_fp8"] * 1e-3) / 1e9, 1),
                              "time_over_tq4": round(q["ms_fp8"] / q["ms_step"], 3)}}
        log(name, json.dumps(legs[name]))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu_baseline: timing the fp64 oracle")
        cpu = cpu_baseline()

    line = {
        "metric": "packed-weight GB/s & TFLOP/s of TQ4_1S dequant-GEMM at M=16 and M=4096",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "dense_m16: TQ4_1S linear, M=16 tokens, K=2688, N=8192, "
                               "W~N(0,0.02^2) packed, x bf16~N(0,1), "
                               f"{args.copies} rotating weight copies",
                   "global_batch": wl.m, "parallelism": "none (1 GPU)",
                   "weight_copies_read_in_timed_steps": min(args.steps, args.copies),
                   "infinity_cache_flushed_before_timing": True},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
