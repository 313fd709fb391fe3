#!/usr/bin/env python
"""Benchmark of the ternary linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sections ...] [--no-cpu]

Headline (the JSON `value`): one prefill step of the gate/up projection,
M=512 tokens, K=5120, N=17408 -- rotate_quant_act followed by ternary_linear
(int8-MFMA GEMM with fused 2-bit unpack and rescale) -- reported as int8 TOPS
(2*M*N*K per step / step time), the steps launched one by one from Python.
The same steps captured once as a HIP graph and replayed (the launch path of
a serving loop) are reported beside it ("ms_per_step_graph"): within a few
percent for this prefill step, whose kernels outlast their launch cost, and
much faster for the small decode steps, where host launch overhead dominates.  Packing is a load-time operation and is done once before
timing.  Inputs are seeded synthetic data with the pages' layer
shapes; weights cycle through enough copies (>= 1.1 GB) that every step reads
them from HBM rather than from the 256 MB last-level cache.

Also measured and printed under "detail": the down projection (M=256,
K=17408, N=5120), the decode sweep M in {1,4,8,16,24} over both layer shapes
(weight GB/s), and the 64-layer stack (one 512-token prefill step and one
24-token decode step), plus each kernel's own time from HIP events.

"roofline" is for the dominant kernel (the prefill GEMM): achieved int8 TOP/s
from its average event-timed duration against the 5.0 POP/s dense int8 MFMA
peak.  "cpu_baseline" times the CPU oracle on the host (rank 0 only) on
repeated full steps of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int8 TOPS (prefill GEMM) + weight GB/s (decode GEMV), ms/step, % of roofline"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
# VALU int8 dot4: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz x 4 MACs x 2 ops
PEAK_VALU_DOT4_TOPS = 256 * 4 * 16 * 2.4e9 * 8 / 1e12
CACHE_BUST_BYTES = int(1.1e9)
COPY_BYTES = 1 << 30
SECTIONS = ("headline", "down", "decode", "stack", "peaks")


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def weight_bytes(N: int, K: int) -> int:
    return N * K // 4 + N * K // 128 + 4 * N


def upload_layer(torch, twl, layer, copies: int):
    """Host layer -> device x, sign and `copies` packed weight sets."""
    x = torch.from_numpy(layer.x_bits.view("int16")).cuda()
    sign = torch.from_numpy(layer.sign).cuda()
    code = torch.from_numpy(layer.code).cuda()
    s = torch.from_numpy(layer.s_bits.view("int16")).cuda()
    packed, q, smax = twl.pack_ternary(code, s)
    del code
    sets = [(packed, q, smax)]
    for _ in range(copies - 1):
        sets.append((packed.clone(), q.clone(), smax.clone()))
    return x, sign, sets


def n_copies(N: int, K: int) -> int:
    return max(1, -(-CACHE_BUST_BYTES // weight_bytes(N, K)))


def graph_time_stats(torch, fn, iters: int = 50, replays: int = 10) -> dict:
    """Per-call GPU time of fn(): `iters` calls are captured into one HIP graph
    (so host launch cost, ~10 us per call from Python, does not count) and the
    graph is replayed `replays` times after 2 untimed replays, each replay
    timed with HIP events on the capture stream.  Returns the median, p10 and
    p90 over the replays of (replay time / iters), in ms, and the number of
    timed calls."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(iters):
            fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        with torch.cuda.stream(s):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / iters)
    del g
    per.sort()

    def q(f):
        return per[min(len(per) - 1, max(0, int(round(f * (len(per) - 1)))))]

    return {"median_ms": q(0.5), "p10_ms": q(0.1), "p90_ms": q(0.9), "calls": iters * replays}


def graph_time_ms(torch, fn, iters: int = 50, replays: int = 10) -> float:
    """Median per-call ms of fn() (graph_time_stats)."""
    return graph_time_stats(torch, fn, iters, replays)["median_ms"]


def _graph_time_best_ms(torch, fn, iters: int, replays: int = 3) -> float:
    """Best-of-replays variant (kept for the peaks microbenchmarks' read calls)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(replays):
        with torch.cuda.stream(s):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        best = ms if best is None else min(best, ms)
    del g
    return best


def event_time_ms(torch, fn, iters: int = 10, warm: int = 3) -> float:
    """Mean ms of fn() over `iters` back-to-back calls, HIP events on the
    current stream (for library calls that are not captured in a graph)."""
    for _ in range(warm):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def pages_int8_path(torch, twl, layer, x, sign, packed_q_smax):
    """The pages' int8 design ([P1] section 4) on the same GPU, as an A/B point:
    expand W_int8 = code * q in HBM every step (plain torch ops), the library
    int8 GEMM (torch._int_mm, hipBLASLt on ROCm; B as a column-major view of
    W_int8), and the per-token / per-row rescale as a torch elementwise pass."""
    import numpy as np
    _, q, smax = packed_q_smax
    code = torch.from_numpy(np.ascontiguousarray(layer.code)).cuda()
    x_i8, a_scale = twl.rotate_quant_act(x, sign)
    q_rep = q.repeat_interleave(128, dim=1)
    expand = lambda: code * q_rep
    w = expand()
    mm = lambda: torch._int_mm(x_i8, w.t())
    acc = mm()
    col = smax * (1.0 / 127.0)
    rescale = lambda: acc.float() * a_scale[:, None] * col[None, :]
    out = {"expand_ms": event_time_ms(torch, expand), "int_mm_ms": event_time_ms(torch, mm),
           "rescale_ms": event_time_ms(torch, rescale)}
    out["total_ms"] = out["expand_ms"] + out["int_mm_ms"] + out["rescale_ms"]
    ops = 2.0 * layer.M * layer.N * layer.K
    out["int_mm_tops"] = round(ops / out["int_mm_ms"] / 1e9, 2)
    out = {k: (round(v, 5) if k.endswith("_ms") else v) for k, v in out.items()}
    del code, q_rep, w, acc
    torch.cuda.empty_cache()
    return out


def run_layer_steps(torch, twl, x, sign, sets, steps, warmup, kernel_iters=50, bf16=False, dot4=False):
    """warmup + timed steps of rotate_quant_act + ternary_linear.

    Returns (ms per step from the wall clock around exactly `steps` eager
    steps, ms per step of the `steps` steps launched as one captured HIP graph
    (median over 5 replays timed with HIP events),
    the per-call time statistics of rotate_quant_act and of ternary_linear, a
    dict of further statistics); the per-call statistics come from HIP events
    around replays of a captured graph of `kernel_iters` back-to-back launches
    of that call alone (weights cycled), see graph_time_stats.  bf16=True adds
    "lin16" (y written in bf16), dot4=True adds "dot4" (the decode path forced
    to the dot4 GEMV).
    """
    M, K = x.shape
    N = sets[0][2].shape[0]
    x_i8 = torch.empty((M, K), dtype=torch.int8, device="cuda")
    a_scale = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws_n = twl.workspace_bytes(M, N, K)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def rotq():
        twl.rotate_quant_act(x, sign, out=(x_i8, a_scale))

    def linear(i):
        packed, q, smax = sets[i % len(sets)]
        twl.ternary_linear(x_i8, a_scale, packed, q, smax, out=y, workspace=ws)

    for i in range(warmup):
        rotq()
        linear(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        rotq()
        linear(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps

    # the same `steps` steps (weights still cycled) captured once as a HIP
    # graph, the way a serving loop launches them; one untimed replay, then
    # the median over 5 replays, each timed with HIP events on the replay
    # stream (a single replay timed by the host clock varied by +-15% here)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(steps):
            rotq()
            linear(i)
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(5):
        with torch.cuda.stream(side):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(side)
            g.replay()
            e1.record(side)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / steps)
    per.sort()
    ms_graph = per[len(per) // 2]
    del g

    rq = graph_time_stats(torch, rotq, kernel_iters)
    ctr = [0]

    def linear_next():
        linear(ctr[0])
        ctr[0] += 1

    lin = graph_time_stats(torch, linear_next, kernel_iters)
    extra = {}
    if bf16:
        y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def linear_bf16_next():
            packed, q, smax = sets[ctr[0] % len(sets)]
            twl.ternary_linear_bf16(x_i8, a_scale, packed, q, smax, out=y16, workspace=ws)
            ctr[0] += 1

        extra["lin16"] = graph_time_stats(torch, linear_bf16_next, kernel_iters)
    if dot4:
        def linear_dot4_next():
            packed, q, smax = sets[ctr[0] % len(sets)]
            twl.ternary_linear(x_i8, a_scale, packed, q, smax, path=twl.PATH_GEMV_DOT4, out=y, workspace=ws)
            ctr[0] += 1

        extra["dot4"] = graph_time_stats(torch, linear_dot4_next, kernel_iters)
    return ms_step, ms_graph, rq, lin, extra


def traffic_for(kernel_src: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    src = os.path.join(ROOT, "ternary_weight_linear_block_amd", "csrc", kernel_src)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for ln in open(path):
        p = ln.split()
        if len(p) >= 5 and not ln.startswith("#") and p[0] == kernel_src and p[1] == workload:
            if p[2] == sha:
                return float(p[3]) + float(p[4])
    return None


def cpu_baseline(layer, min_s=12.0, max_reps=400):
    """The CPU oracle as it stands, on repeated full steps of the workload."""
    import numpy as np
    import oracle.twl_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    q, smax = O.decompose_scales(layer.s_bits)     # load time, outside the timing
    reps = 0
    t0 = time.perf_counter()
    while True:
        x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
        y = O.ternary_linear(x_i8, a_scale, layer.code, q, smax)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s or reps >= max_reps:
            break
    ops = 2.0 * layer.M * layer.N * layer.K * reps
    del y
    return {"value": round(ops / el / 1e12, 4), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full steps (rotate_quant_act + ternary_linear, M={layer.M} K={layer.K} "
                      f"N={layer.N}) in {el:.1f} s; numpy, BLAS threads={threads}, "
                      f"affine cores={len(os.sched_getaffinity(0))}, cpu={cpu_model()}"}


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (empty if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def copy_calibration(torch) -> int:
    """y = -x over COPY_BYTES of float32: each launch reads and writes exactly
    COPY_BYTES, the known size that HBM byte counters are scaled against."""
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES,
                      "copy_calibration_bytes_written": COPY_BYTES, "launches": 3}), flush=True)
    return 0


def kernel_only(torch, twl, name, launches, decode_m) -> int:
    """Launches ternary_linear alone on one workload `launches` times (weights
    cycled through the cache-busting copies, inputs resident), for rocprofv3
    runs; prints the plan and the launch count."""
    import workloads as W
    layer = W.make_config(name)
    x, sign, sets = upload_layer(torch, twl, layer, n_copies(layer.N, layer.K))
    M = decode_m if name.startswith("decode") else layer.M
    x = x[:M].contiguous()
    x_i8, a_scale = twl.rotate_quant_act(x, sign)
    y = torch.empty((M, layer.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, twl.workspace_bytes(M, layer.N, layer.K)), dtype=torch.uint8, device="cuda")
    for i in range(launches):
        packed, q, smax = sets[i % len(sets)]
        twl.ternary_linear(x_i8, a_scale, packed, q, smax, out=y, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": name, "M": M, "K": layer.K, "N": layer.N, "launches": launches,
                      "plan": twl.plan_info(M, layer.N, layer.K)}), flush=True)
    return 0


def section_layer(torch, twl, name, steps, warmup):
    import numpy as np
    import workloads as W
    layer = W.make_config(name)
    x, sign, sets = upload_layer(torch, twl, layer, n_copies(layer.N, layer.K))
    ms, ms_graph, rqs, lins, ex = run_layer_steps(torch, twl, x, sign, sets, steps, warmup, bf16=True)
    rq, lin, lin16 = rqs["median_ms"], lins["median_ms"], ex["lin16"]["median_ms"]
    ops = 2.0 * layer.M * layer.N * layer.K
    extra = {}
    if name == "prefill_gate_up":
        # the bf16 reference path ([P1] section 4's pre-int8 path) on the same
        # layer: the rotation to bf16, then the exact-dequant bf16 MFMA kernel
        # (one weight copy: this is an A/B point, not the hot path)
        s_d = torch.from_numpy(layer.s_bits.view(np.int16)).cuda()
        packed0 = sets[0][0]
        r = twl.rotate_act_bf16(x, sign)
        yr = torch.empty((layer.M, layer.N), dtype=torch.float32, device="cuda")
        rot_ms = graph_time_ms(torch, lambda: twl.rotate_act_bf16(x, sign, out=r), 20)
        ref_ms = graph_time_ms(torch, lambda: twl.reference_linear_bf16(r, packed0, s_d, out=yr), 5)
        extra = {"reference_bf16_rotate_ms": round(rot_ms, 5), "reference_bf16_linear_ms": round(ref_ms, 5),
                 "reference_bf16_tflops": round(ops / ref_ms / 1e9, 2)}
        del r, yr, s_d
        extra["pages_int8_path"] = pages_int8_path(torch, twl, layer, x, sign, sets[0])
    if layer.act == "silu_gate":
        # the fused SiLU(gate) * up + rotation of this layer's input, from a
        # [M, 2K] gate/up tensor (random bf16, drawn on the GPU)
        g = torch.Generator(device="cuda").manual_seed(7)
        gu = torch.randn((layer.M, 2 * layer.K), generator=g, device="cuda").to(torch.bfloat16)
        xi = torch.empty((layer.M, layer.K), dtype=torch.int8, device="cuda")
        sc = torch.empty((layer.M,), dtype=torch.float32, device="cuda")
        fused = graph_time_ms(torch, lambda: twl.silu_mul_rotate_quant_act(gu, sign, out=(xi, sc)), 50)
        fb = layer.M * layer.K * 5 + layer.M * 4 + layer.K
        extra = {"silu_rotq_ms": round(fused, 5), "silu_rotq_gbs": round(fb / fused / 1e6, 1)}
        del gu
    out = {"M": layer.M, "K": layer.K, "N": layer.N, "ms_per_step": round(ms, 5),
           "step_tops": round(ops / ms / 1e9, 2), "ms_per_step_graph": round(ms_graph, 5),
           "step_tops_graph": round(ops / ms_graph / 1e9, 2), "linear_ms": round(lin, 5),
           "linear_p10_ms": round(lins["p10_ms"], 5), "linear_p90_ms": round(lins["p90_ms"], 5),
           "linear_calls_timed": lins["calls"], "linear_tops": round(ops / lin / 1e9, 2),
           "linear_plan": twl.plan_info(layer.M, layer.N, layer.K),
           "linear_bf16_y_ms": round(lin16, 5), "linear_bf16_y_tops": round(ops / lin16 / 1e9, 2),
           "rotq_ms": round(rq, 5), "rotq_p10_ms": round(rqs["p10_ms"], 5), "rotq_p90_ms": round(rqs["p90_ms"], 5),
           "rotq_gbs": round((layer.M * layer.K * 3 + layer.M * 4 + layer.K) / rq / 1e6, 1),
           "weight_copies": len(sets), **extra}
    del sets, x
    torch.cuda.empty_cache()
    return layer, out


def fused_stats(torch, twl, x, sign, sets, iters: int = 50) -> dict:
    """Per-call time of rotate_quant_linear (the rotation and the decode kernel
    fused into one launch) from bf16 x, weights cycled, as graph_time_stats."""
    M, K = x.shape
    N = sets[0][2].shape[0]
    x_i8 = torch.empty((M, K), dtype=torch.int8, device="cuda")
    a_scale = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ctr = [0]

    def call():
        packed, q, smax = sets[ctr[0] % len(sets)]
        ctr[0] += 1
        twl.rotate_quant_linear(x, sign, packed, q, smax, out=y, x_i8=x_i8, a_scale=a_scale)
    return graph_time_stats(torch, call, iters)


def section_decode(torch, twl, steps, warmup):
    import workloads as W
    res = {}
    for name in ("decode_gate_up", "decode_down"):
        layer = W.make_config(name)
        x_full, sign, sets = upload_layer(torch, twl, layer, n_copies(layer.N, layer.K))
        per_m = {}
        for M in W.DECODE_MS:
            x = x_full[:M].contiguous()
            ms, ms_graph, rqs, lins, ex = run_layer_steps(torch, twl, x, sign, sets, steps, warmup, dot4=True)
            lin, d4 = lins["median_ms"], ex["dot4"]["median_ms"]
            wb = weight_bytes(layer.N, layer.K)
            tot = wb + M * layer.K + M * 4 + 4 * M * layer.N
            ops = 2.0 * M * layer.N * layer.K
            plan = twl.plan_info(M, layer.N, layer.K)
            per_m[str(M)] = {"ms_per_step": round(ms, 5), "ms_per_step_graph": round(ms_graph, 5),
                             "kernel": plan["family"],
                             "linear_ms": round(lin, 5), "linear_p10_ms": round(lins["p10_ms"], 5),
                             "linear_p90_ms": round(lins["p90_ms"], 5), "linear_calls_timed": lins["calls"],
                             "weight_gbs": round(wb / lin / 1e6, 1),
                             "hbm_frac": round(wb / lin / 1e6 / PEAK_HBM_GBS, 4),
                             "total_gbs": round(tot / lin / 1e6, 1),
                             "tops": round(ops / lin / 1e9, 2),
                             "mfma_frac": round(ops / lin / 1e9 / PEAK_INT8_TOPS, 5),
                             "dot4_ms": round(d4, 5), "dot4_p10_ms": round(ex["dot4"]["p10_ms"], 5),
                             "dot4_p90_ms": round(ex["dot4"]["p90_ms"], 5),
                             "dot4_weight_gbs": round(wb / d4 / 1e6, 1),
                             "dot4_hbm_frac": round(wb / d4 / 1e6 / PEAK_HBM_GBS, 4),
                             "dot4_tops": round(ops / d4 / 1e9, 2),
                             "rotq_ms": round(rqs["median_ms"], 5), "rotq_p10_ms": round(rqs["p10_ms"], 5),
                             "rotq_p90_ms": round(rqs["p90_ms"], 5)}
            if twl.rotate_quant_linear_fused(M, layer.N, layer.K):
                # the same step as one fused launch (rotate_quant_linear)
                fz = fused_stats(torch, twl, x, sign, sets)
                per_m[str(M)].update({"fused_step_ms": round(fz["median_ms"], 5),
                                      "fused_step_p10_ms": round(fz["p10_ms"], 5),
                                      "fused_step_p90_ms": round(fz["p90_ms"], 5),
                                      "fused_weight_gbs": round(wb / fz["median_ms"] / 1e6, 1)})
        res[name] = {"K": layer.K, "N": layer.N, "by_M": per_m}
        del sets, x_full
        torch.cuda.empty_cache()
    return res


def section_stack(torch, twl, steps, warmup):
    """64 decoder layers x {proj 5120->5120, gate_up 5120->34816, down 17408->5120},
    one 512-token prefill step and one 24-token decode step, each run two ways:
      "independent": every linear's input is a pre-drawn activation (rotation
        + linear per linear, 6 launches per layer);
      "chained": the down projection takes its input from the gate/up
        projection of the same layer -- gate/up writes y in bf16 and
        silu_mul_rotate_quant_act turns it into the down projection's int8
        input (also 6 launches per layer).
    Each is timed eagerly (launches from Python) and as one captured HIP graph."""
    import workloads as W
    signs = {k: torch.from_numpy(v).cuda() for k, v in W.stack_signs().items()}
    layers = []
    for L in range(W.N_LAYERS):
        lin = []
        for which in range(3):
            xb, code, s = W.stack_linear_torch(L, which, 512, "cuda")
            packed, q, smax = twl.pack_ternary(code, s)
            del code
            lin.append((xb, packed, q, smax))
        layers.append(lin)
    torch.cuda.synchronize()
    inter = W.STACK_LINEARS[2][1]  # 17408: the down projection's input width
    out = {}
    for M in (512, 24):
        bufs = {}
        for which, (_, K, N, _, _) in enumerate(W.STACK_LINEARS):
            bufs[which] = (torch.empty((M, K), dtype=torch.int8, device="cuda"),
                           torch.empty((M,), dtype=torch.float32, device="cuda"),
                           torch.empty((M, N), dtype=torch.float32, device="cuda"),
                           torch.empty(max(1, twl.workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda"))
        gu16 = torch.empty((M, 2 * inter), dtype=torch.bfloat16, device="cuda")
        xs = [[lin[w][0][:M].contiguous() for w in range(3)] for lin in layers]

        def step_independent():
            for L, lin in enumerate(layers):
                for which, (_, packed, q, smax) in enumerate(lin):
                    K = W.STACK_LINEARS[which][1]
                    x_i8, a_scale, y, ws = bufs[which]
                    twl.rotate_quant_act(xs[L][which], signs[K], out=(x_i8, a_scale))
                    twl.ternary_linear(x_i8, a_scale, packed, q, smax, out=y, workspace=ws)

        def step_chained():
            for L, lin in enumerate(layers):
                for which in (0, 1):
                    _, packed, q, smax = lin[which]
                    K = W.STACK_LINEARS[which][1]
                    x_i8, a_scale, y, ws = bufs[which]
                    twl.rotate_quant_act(xs[L][which], signs[K], out=(x_i8, a_scale))
                    if which == 0:
                        twl.ternary_linear(x_i8, a_scale, packed, q, smax, out=y, workspace=ws)
                    else:
                        twl.ternary_linear_bf16(x_i8, a_scale, packed, q, smax, out=gu16, workspace=ws)
                _, packed, q, smax = lin[2]
                x_i8, a_scale, y, ws = bufs[2]
                twl.silu_mul_rotate_quant_act(gu16, signs[inter], out=(x_i8, a_scale))
                twl.ternary_linear(x_i8, a_scale, packed, q, smax, out=y, workspace=ws)

        ops = 2.0 * M * sum(N * K for _, K, N, _, _ in W.STACK_LINEARS) * W.N_LAYERS
        wb = sum(weight_bytes(N, K) for _, K, N, _, _ in W.STACK_LINEARS) * W.N_LAYERS
        rec = {"launches": 6 * W.N_LAYERS}
        for mode, step in (("independent", step_independent), ("chained", step_chained)):
            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step()
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            ms_graph = (time.perf_counter() - t0) * 1e3 / steps
            del g
            rec[mode] = {"ms_per_step": round(ms, 4), "tops": round(ops / ms / 1e9, 2),
                         "weight_gbs": round(wb / ms / 1e6, 1), "ms_per_step_graph": round(ms_graph, 4),
                         "tops_graph": round(ops / ms_graph / 1e9, 2),
                         "weight_gbs_graph": round(wb / ms_graph / 1e6, 1)}
        # the previous keys: the independent-input step
        rec.update({k: rec["independent"][k] for k in rec["independent"]})
        out["prefill_M512" if M == 512 else "decode_M24"] = rec
        del xs, bufs, gu16
    del layers
    torch.cuda.empty_cache()
    return out


def section_peaks(torch):
    """Measured peaks of this part, from the microbenchmark kernels of
    libtwl_peaks.so, timed with HIP events on the stream they run on: the
    int8 MFMA rate (the GEMM's instruction with no memory traffic), the HBM
    read rate (nontemporal stream of 1 GiB), the time of one streaming read of
    the decode weight size (22.3 MB, graph-captured back to back like the
    decode calls), the VALU v_dot4 int8 rate, and the rate of the prefill
    GEMM's MFMA + 2-bit unpack instruction mix without memory traffic (each
    unpacked operand feeding 2 or 4 MFMAs)."""
    import ctypes
    from ternary_weight_linear_block_amd.build import PEAKS_LIB_PATH
    if not os.path.exists(PEAKS_LIB_PATH):
        raise ImportError(f"{PEAKS_LIB_PATH} is missing: build it first "
                          "(python -m ternary_weight_linear_block_amd.build)")
    lib = ctypes.CDLL(PEAKS_LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.twl_peak_mfma_i8.argtypes = [I, I, P, P]
    lib.twl_peak_read.argtypes = [P, S, I, P, P]
    lib.twl_peak_dot4.argtypes = [I, I, P, P]
    lib.twl_peak_mix_i8.argtypes = [I, I, I, P, P]
    for f in (lib.twl_peak_mfma_i8, lib.twl_peak_read, lib.twl_peak_dot4, lib.twl_peak_mix_i8):
        f.restype = I
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: HIP error {rc}")

    wgs, iters = 1024, 2000
    ms = timed(lambda: check(lib.twl_peak_mfma_i8(wgs, iters, sink.data_ptr(), h), "mfma peak"))
    mfma_tops = 2.0 * 32 * 32 * 32 * 10 * iters * wgs * 4 / (ms * 1e-3) / 1e12
    # the GEMM's MFMA + unpack mix, one workgroup per CU: 3 waves per SIMD
    # with 2 x 3 fragments (reuse 2), 2 waves per SIMD with 4 x 2 (reuse 4)
    mix = {}
    for reuse, frags, wps in ((2, 6, 3), (4, 8, 2)):
        ms = timed(lambda: check(lib.twl_peak_mix_i8(reuse, 256, iters, sink.data_ptr(), h), "mix peak"))
        mix[reuse] = 2.0 * 32 * 32 * 32 * frags * iters * 256 * 4 * wps / (ms * 1e-3) / 1e12
    ms = timed(lambda: check(lib.twl_peak_dot4(wgs, iters, sink.data_ptr(), h), "dot4 peak"))
    dot4_tops = 8.0 * 8 * iters * wgs * 256 / (ms * 1e-3) / 1e12
    big = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    ms = timed(lambda: check(lib.twl_peak_read(big.data_ptr(), COPY_BYTES, 8192, sink.data_ptr(), h),
                             "read peak"))
    read_gbs = COPY_BYTES / (ms * 1e-3) / 1e9
    # one decode-sized read per launch, 48 launches over distinct buffers
    wb = weight_bytes(17408, 5120) // 16 * 16
    copies = 48
    step = (wb + 4095) // 4096 * 4096
    pool = torch.empty(step * copies, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    it = [0]

    def one():
        # on the stream current at call time: graph_time_ms captures on its own
        k = it[0] % copies
        it[0] += 1
        check(lib.twl_peak_read(pool.data_ptr() + k * step, wb, 2048, sink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream), "read call")

    call_ms = _graph_time_best_ms(torch, one, copies)
    del big, pool
    torch.cuda.empty_cache()
    return {"int8_mfma_tops": round(mfma_tops, 1), "int8_mfma_frac_of_spec": round(mfma_tops / PEAK_INT8_TOPS, 4),
            "hbm_read_gbs": round(read_gbs, 1), "hbm_read_frac_of_spec": round(read_gbs / PEAK_HBM_GBS, 4),
            "decode_size_read_us": round(call_ms * 1e3, 2), "decode_size_read_bytes": wb,
            "valu_dot4_tops": round(dot4_tops, 1),
            "mfma_unpack_mix_reuse2_tops": round(mix[2], 1), "mfma_unpack_mix_reuse4_tops": round(mix[4], 1)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="ternary linear layer benchmark (one MI355X)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma list of: " + ", ".join(SECTIONS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--kernel-only", default=None,
                    help="only launch ternary_linear on one workload (prefill_gate_up, prefill_down, "
                         "decode_gate_up, decode_down) --launches times, weights cycled, and exit: "
                         "the run that rocprofv3 counter passes profile")
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--decode-m", type=int, default=1, help="tokens for --kernel-only decode_*")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a copy-like kernel of known traffic (y = -x over 1 GiB of "
                         "float32, 3 launches) to scale HBM byte counters, then exit")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU only (no collectives, no sharding); "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import ternary_weight_linear_block_amd as twl
    twl.library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(torch)
    if args.kernel_only:
        return kernel_only(torch, twl, args.kernel_only, args.launches, args.decode_m)
    sections = [s for s in args.sections.split(",") if s]
    detail = {"device": torch.cuda.get_device_name(0)}

    log("headline: prefill gate/up M=512 K=5120 N=17408")
    layer, head = section_layer(torch, twl, "prefill_gate_up", args.steps, args.warmup)
    detail["prefill_gate_up"] = head
    if "down" in sections:
        log("prefill down M=256 K=17408 N=5120")
        detail["prefill_down"] = section_layer(torch, twl, "prefill_down", args.steps, args.warmup)[1]
    if "decode" in sections:
        log("decode sweep")
        detail["decode"] = section_decode(torch, twl, args.steps, args.warmup)
    if "stack" in sections:
        log("64-layer stack")
        detail["stack"] = section_stack(torch, twl, max(2, args.steps // 10), 1)
    peaks = None
    if "peaks" in sections:
        log("measured peaks (microbenchmarks)")
        peaks = section_peaks(torch)
        detail["measured_peaks"] = peaks

    ops = 2.0 * layer.M * layer.N * layer.K
    achieved = ops / head["linear_ms"] / 1e9
    plan = head["linear_plan"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                "traffic": traffic_for("gemm_i8.hip", "prefill_gate_up"),
                "kernel": f"gemm_kernel ({plan['tile_rows']}x{plan['tile_cols']} tiles, "
                          f"{plan['workgroups']} workgroups, ternary_linear GEMM path)",
                "algorithmic_ops_per_launch": ops,
                "launch_ms_median": head["linear_ms"], "launch_ms_p10": head["linear_p10_ms"],
                "launch_ms_p90": head["linear_p90_ms"], "launches_timed": head["linear_calls_timed"]}
    if peaks:
        roofline["measured_peak"] = peaks["int8_mfma_tops"]
        roofline["frac_of_measured_peak"] = round(achieved / peaks["int8_mfma_tops"], 4)
    decode_roofline = None
    if "decode" in detail:
        # the decode kernel the automatic path takes, against HBM on its
        # algorithmic weight bytes (the metric's weight GB/s); the forced dot4
        # GEMV beside it against the measured v_dot4 rate
        dot4_peak = peaks["valu_dot4_tops"] if peaks else PEAK_VALU_DOT4_TOPS
        by = {}
        for lname, rec_l in detail["decode"].items():
            for m, r in rec_l["by_M"].items():
                r["dot4_valu_frac"] = round(r["dot4_tops"] / dot4_peak, 4)
                by[f"{lname} M={m}"] = {"kernel": r["kernel"], "weight_gbs": r["weight_gbs"],
                                        "frac": r["hbm_frac"], "dot4_weight_gbs": r["dot4_weight_gbs"],
                                        "dot4_valu_frac": r["dot4_valu_frac"]}
                if "fused_step_ms" in r:
                    by[f"{lname} M={m}"]["fused_step_ms"] = r["fused_step_ms"]
        g1 = detail["decode"]["decode_gate_up"]["by_M"]["1"]
        dl = detail["decode"]["decode_gate_up"]
        decode_roofline = {"bound": "hbm", "kernel": "gemv_rows_kernel (decode path, M <= 24)",
                           "workload": f"decode_gate_up M=1 K={dl['K']} N={dl['N']}",
                           "achieved": g1["weight_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": g1["hbm_frac"], "algorithmic_bytes_per_launch": weight_bytes(dl["N"], dl["K"]),
                           "traffic": traffic_for("gemv.hip", "decode_gate_up_m1"),
                           "dot4_peak_tops": dot4_peak, "by_layer_and_M": by}
    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(layer)

    rec = {"metric": METRIC, "value": head["step_tops"], "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
           "data": "synthetic",
           "config": {"workload": "prefill_gate_up", "M": layer.M, "K": layer.K, "N": layer.N,
                      "step": "rotate_quant_act + ternary_linear",
                      "launch": "eager (graph-launched figure in detail)",
                      "parallelism": "none (1 GPU)"},
           "roofline": roofline, "decode_roofline": decode_roofline, "cpu_baseline": cpu, "detail": detail}
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
