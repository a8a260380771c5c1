#!/usr/bin/env python3
"""Throughput of the FP8 blockwise linear layer on one MI355X (gfx950).

A step is one forward pass of the linear layer over one batch of synthetic
activations already resident in HBM: the activation quantizer (fused with
RMSNorm for the prefill-with-norm workload, and with the residual add in front
of it for the add-norm workload, which updates the stream in place) followed
by the scaled GEMM (`*_pow2` workloads: the same with power-of-two scales
-- block FP8 as an MXFP8 view -- applied inside the MFMA; `decode_splitk`:
the split-K entry point with its workspace; `moe_*`: the
expert-sorted rows of one GPU's share of a MoE layer through the grouped
GEMM).  The
weight is quantized once before timing (it is offline preparation).  Inputs,
outputs and weight copies rotate over several buffer sets whose total exceeds
the 256 MB Infinity Cache, so HBM rates are not inflated by cache hits.

Prints ONE JSON line.  `value` = 2*M*N*K per step / step time (whole layer,
quantizer included), the steps timed without anything recorded between
their launches.  Kernel launch durations are measured two ways with HIP
events recorded on the kernel's stream: inside the steps (`us_in_step`:
events around each launch in a second pass of the same steps, the dispatch
gap before the launch included) and over back-to-back launches (captured
once in a HIP graph and replayed, so that a short kernel is not timed at the
host's launch rate; each launch meets the previous one's output
write-back).  `roofline` is for the dominant kernel (the GEMM) at the
tighter of its two durations (`kernel_timing` says which); the quantizer's
rate is from back-to-back launches.  For workloads with the RMSNorm front
end, `quant_group` is the group quantizer alone over the same activations
(not part of a step); `cpu_baseline` is the CPU oracle timed on a bounded
sample of the same workload on this host.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-FP8 GEMM TFLOP/s & % FP8 MFMA peak; group-quant HBM GB/s"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, 5.0 PFLOP/s
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, 8 TB/s
MALL_DEFEAT_BYTES = 640 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~20 ms of warm-up steps (the chip reaches its steady clock
    # only after some tens of milliseconds of sustained load; 10 warm-up
    # steps left the first timed steps ~20 % slower) and ~20 ms timed
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_norm",
                    choices=["tiny", "decode", "prefill_norm", "prefill_addnorm", "large", "mx", "pertensor",
                             "prefill_norm_pow2", "large_pow2", "moe_up", "moe_down", "decode_splitk"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (0 = skip)")
    return ap.parse_args()


def code_text(src: str) -> str:
    """C/C++ source without its comments, trailing blanks and empty lines
    (string and character literals kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


# sources that do not build the GEMM kernels (whose traffic the counters give)
NON_GEMM_SOURCES = {"quant_kernels.hip"}


def kernel_source_sha(csrc: str | None = None) -> str:
    """Hash of the code of the sources the GEMM kernels are built from (every
    source but the quantizers'; comments and blank lines excluded, so that a
    change of documentation keeps the counters taken before it)."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "fp8_block_scaled_token_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f in NON_GEMM_SOURCES:
            continue
        h.update(f.encode())
        h.update(code_text(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """L2<->fabric bytes per GEMM launch (FETCH_SIZE and WRITE_SIZE, scaled by
    a device copy) from committed rocprofv3 counters, or None
    when the GEMM kernels have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    rec = t.get("workloads", {}).get(workload)
    return None if rec is None else rec.get("traffic_bytes")



SETTLE_MS = 60.0


def settle_clocks(step, budget_ms=SETTLE_MS):
    """Run `step(i)` (untimed) until at least budget_ms of GPU time has passed.

    The GPU's clocks ramp up over the first ~25 ms of sustained load (the same
    kernel runs ~20 % slower there), so a few warm-up steps alone leave the
    timed region on a cold clock.  This is part of the warm-up: nothing it
    runs is timed or reported."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    i, spent = 0, 0.0
    while spent < budget_ms and i < 100000:
        for _ in range(8):
            step(i)
            i += 1
        e1.record()
        e1.synchronize()
        spent = e0.elapsed_time(e1)
    torch.cuda.synchronize()


def launch_ms(fn, sets, reps, stream, record):
    """Mean duration of one launch of fn over `reps` back-to-back launches
    (rotating buffer sets), from HIP events recorded on the launch stream.
    The launches are captured once in a HIP graph and the graph is replayed,
    so that a kernel shorter than the host's launch interval is timed on the
    GPU's clock rather than at the host's launch rate; if capture fails the
    launches are issued eagerly.  `record["kernel_timing"]` says which."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = len(sets)
    settle_clocks(lambda i: fn(sets[i % n]))
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(graph, stream=side):
            for i in range(reps):
                fn(sets[i % n])
        torch.cuda.synchronize()
        graph.replay()                               # first replay: warm
        torch.cuda.synchronize()
        # a replay in flight while the timed one is submitted, so that the
        # GPU reaches e0 with the timed replay's launches already queued (the
        # host's submission time stays outside the interval)
        graph.replay()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        record.setdefault("kernel_timing", "graph replay of back-to-back launches")
        del graph
        return e0.elapsed_time(e1) / reps
    except RuntimeError:
        torch.cuda.synchronize()
        record["kernel_timing"] = "eager back-to-back launches (graph capture failed)"
    e0.record(stream)
    for i in range(reps):
        fn(sets[i % n])
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps

def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1; sharding is described in DESIGN.md)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp8_block_scaled_token_amd as fq
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    fq.load_library()

    name = args.workload
    if name in workloads.MOE_WORKLOADS:
        return moe_main(args, workloads.MOE_WORKLOADS[name])
    pow2 = name.endswith("_pow2")
    wl = workloads.WORKLOADS["mx" if name == "pertensor" else name[:-5] if pow2 else name]
    M, N, K = wl.M, wl.N, wl.K
    d = wl.make("cpu")
    x_cpu, w_cpu = d["x"], d["w"]
    KB, NB = math.ceil(K / 128), math.ceil(N / 128)

    # ---- weights: quantized once (offline preparation, not timed)
    wd = w_cpu.cuda()
    if name == "mx":
        # MX scales column-major ([K/32, rows]), the layout the GEMM reads as
        # contiguous runs; the weight's rows are quantized like activations
        qw, sw = fq.quant_act_mx(wd, layout=fq.COL_MAJOR)
    elif name == "pertensor":
        qw, sw = fq.quant_weight_tensor(wd)
    elif pow2:
        # a block-FP8 checkpoint re-expressed with power-of-two block scales
        qw, sw = fq.requant_weight_pow2(*fq.quant_weight_block(wd))
    else:
        qw, sw = fq.quant_weight_block(wd)
    gamma = d["gamma"].cuda() if wl.norm else None
    del wd
    sx_static = None
    if name == "pertensor":
        amax = float(x_cpu.float().abs().max())
        sx_static = torch.tensor([np.float32(np.float32(amax) / np.float32(448.0))], device="cuda")

    # ---- rotating activation / output sets (beat the Infinity Cache)
    set_bytes = M * K * 2 + M * K + M * KB * 4 + M * N * 2 + (M * K * 2 if wl.residual else 0)
    nsets = max(1, min(8, math.ceil(MALL_DEFEAT_BYTES / set_bytes)))
    xg = x_cpu.cuda()
    hg = d["h"].cuda() if wl.residual else None
    sets = []
    for _ in range(nsets):
        s = {"x": xg.clone(), "q": torch.empty(M, K, dtype=torch.uint8, device="cuda")}
        if wl.residual:
            s["h"] = hg.clone()
        if name == "mx":
            s["s"] = torch.empty(math.ceil(K / 32), M, dtype=torch.uint8, device="cuda")
        elif name == "pertensor":
            s["s"] = sx_static
        else:
            s["s"] = torch.empty(KB, M, dtype=torch.float32, device="cuda")
        s["y"] = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        sets.append(s)
    del xg, hg

    # ---- weight copies: a weight must not stay in the Infinity Cache between
    # its uses either (a decode weight is 151 MB), so the sets rotate over
    # enough copies that several hundred MB lie between two uses of one copy
    w_bytes = qw.numel() * qw.element_size() + sw.numel() * sw.element_size()
    nw = max(1, min(nsets, math.ceil(MALL_DEFEAT_BYTES / w_bytes)))
    wcopies = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(nw - 1)]
    for i, s in enumerate(sets):
        s["qw"], s["sw"] = wcopies[i % nw]

    # activation group scales travel column-major ([K/128, M]): a K block's
    # scales for consecutive rows are contiguous, one cache line per 32 rows
    # for the GEMM (the row-major form costs a line per row)
    def quant(s):
        if pow2 and wl.norm:
            fq.fp8q_add_rmsnorm_quant(s["x"], None, None, gamma, d["eps"], fq.SCALE_F32_POW2, fq.COL_MAJOR, None,
                                      s["q"], s["s"])
        elif pow2:
            fq.fp8q_quant_act_group(s["x"], 128, fq.SCALE_F32_POW2, fq.COL_MAJOR, None, s["q"], s["s"])
        elif wl.residual:
            fq.fp8q_add_rmsnorm_quant(s["x"], s["h"], s["x"], gamma, d["eps"], fq.SCALE_F32, fq.COL_MAJOR, None,
                                      s["q"], s["s"])
        elif wl.norm:
            fq.fp8q_rmsnorm_quant(s["x"], gamma, d["eps"], fq.COL_MAJOR, s["q"], s["s"])
        elif name == "mx":
            fq.fp8q_quant_act_group(s["x"], 32, fq.SCALE_UE8M0, fq.COL_MAJOR, None, s["q"], s["s"])
        elif name == "pertensor":
            fq.fp8q_quant_act_group(s["x"], 128, fq.SCALE_F32, fq.ROW_MAJOR, sx_static, s["q"], None)
        else:
            fq.fp8q_quant_act_group(s["x"], 128, fq.SCALE_F32, fq.COL_MAJOR, None, s["q"], s["s"])

    # the split entry with its workspace (allocated once by the caller):
    # decode shapes that leave CUs idle split K; prefill shapes split the
    # leftover tiles of their last round along K
    ws = None
    ws_bytes = fq.fp8q_gemm_splitk_workspace_size(M, N, K) if name != "mx" else 0
    if ws_bytes:
        ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")

    def gemm(s):
        if ws is not None:
            gran = {"pertensor": fq.GRAN_PER_TENSOR}.get(name, fq.GRAN_BLOCK128_POW2 if pow2 else fq.GRAN_BLOCK128)
            layout = fq.ROW_MAJOR if name == "pertensor" else fq.COL_MAJOR
            fq.fp8q_gemm_blockscale_splitk(s["q"], s["s"], layout, s["qw"], s["sw"], None, s["y"], gran, ws)
        elif name == "mx":
            fq.fp8q_gemm_mxfp8(s["q"], s["s"], s["qw"], s["sw"], None, s["y"], fq.COL_MAJOR)
        elif name == "pertensor":
            fq.fp8q_gemm_blockscale(s["q"], s["s"], fq.ROW_MAJOR, s["qw"], s["sw"], None, s["y"], fq.GRAN_PER_TENSOR)
        else:
            fq.fp8q_gemm_blockscale(s["q"], s["s"], fq.COL_MAJOR, s["qw"], s["sw"], None, s["y"],
                                    fq.GRAN_BLOCK128_POW2 if pow2 else fq.GRAN_BLOCK128)

    def step(i):
        s = sets[i % nsets]
        quant(s)
        gemm(s)

    settle_clocks(step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps

    # Each kernel's share of a step, from HIP events around the two launches,
    # in a second pass of the same steps after the timed region (recording
    # events inside the timed steps would add their own cost to the step).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        s = sets[i % nsets]
        ev[i][0].record(stream)
        quant(s)
        ev[i][1].record(stream)
        gemm(s)
        ev[i][2].record(stream)
    torch.cuda.synchronize()

    # Launch durations, both ways measured with HIP events on the kernel's
    # stream: inside the steps (events around each launch; the dispatch gap
    # after the previous kernel included) and over back-to-back launches
    # (rotating buffer sets, so inputs still come from HBM; each launch then
    # meets the previous one's output write-back).  Each bounds the kernel's
    # duration from above; the roofline takes the tighter one: inside the
    # steps for a long GEMM, back to back where the dispatch gap is a large
    # share of a short kernel.
    def timed(fn, reps):
        return launch_ms(fn, sets, reps, stream, timing)

    timing = {}
    reps = max(args.steps, 2 * nsets)
    quant_ms = timed(quant, reps)
    gemm_b2b_ms = timed(gemm, reps)
    step_quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    step_gemm_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    gemm_ms = min(step_gemm_ms, gemm_b2b_ms)
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12

    # algorithmic bytes
    if name == "mx":
        q_bytes = M * K * 2 + M * K + M * math.ceil(K / 32)
        g_bytes = M * K + N * K + (M + N) * math.ceil(K / 32) + 2 * M * N
    elif name == "pertensor":
        q_bytes = M * K * 2 + M * K
        g_bytes = M * K + N * K + 8 + 2 * M * N
    else:
        q_bytes = M * K * 2 + M * K + 4 * M * KB + (2 * K if wl.norm else 0) + (4 * M * K if wl.residual else 0)
        g_bytes = M * K + N * K + 4 * M * KB + 4 * NB * KB + 2 * M * N
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    gemm_gbps = g_bytes / (gemm_ms * 1e-3) / 1e9
    quant_gbps = q_bytes / (quant_ms * 1e-3) / 1e9
    hbm_bound = M <= 64
    traffic = measured_traffic(name)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gemm_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gemm_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic}

    kernel_q = {"prefill_norm": "rmsnorm_quant", "prefill_addnorm": "add_rmsnorm_quant", "mx": "quant_group32mx",
                "pertensor": "quant_static", "prefill_norm_pow2": "rmsnorm_quant (pow2 scales)",
                "large_pow2": "quant_group128 (pow2 scales)"}.get(name, "quant_group128")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K, "norm": wl.norm, "residual_add": wl.residual,
                   "scales": {"mx": "1x32 ue8m0, [K/32, rows]", "pertensor": "per-tensor fp32"}.get(
                       name, "group128 + 128x128 power-of-two fp32 (in-MFMA)" if pow2 else "group128 + 128x128 fp32"),
                   "rotating_buffer_sets": nsets, "weight_copies": nw, "splitk_workspace_bytes": ws_bytes},
        "roofline": roof,
        "gemm": {"us": round(gemm_ms * 1e3, 2), "TFLOP/s": round(gemm_tflops, 1),
                 "frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "GB/s": round(gemm_gbps, 1),
                 "algorithmic_bytes": g_bytes, "us_in_step": round(step_gemm_ms * 1e3, 2),
                 "us_back_to_back": round(gemm_b2b_ms * 1e3, 2)},
        "quant": {"kernel": kernel_q, "us": round(quant_ms * 1e3, 2), "GB/s": round(quant_gbps, 1),
                  "frac_hbm": round(quant_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": q_bytes,
                  "us_in_step": round(step_quant_ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    out["kernel_timing"] = {"gemm": "in the steps" if step_gemm_ms <= gemm_b2b_ms else timing.get("kernel_timing"),
                            "quant": timing.get("kernel_timing")}
    if wl.norm and not pow2:
        # the group quantizer on its own (no norm in front) over the same
        # activations, for its HBM fraction on this shape; not part of a step
        def quant_plain(s):
            fq.fp8q_quant_act_group(s["x"], 128, fq.SCALE_F32, fq.COL_MAJOR, None, s["q"], s["s"])
        qp_ms = timed(quant_plain, reps)
        qp_bytes = M * K * 2 + M * K + 4 * M * KB
        qp_gbps = qp_bytes / (qp_ms * 1e-3) / 1e9
        out["quant_group"] = {"kernel": "quant_group128", "us": round(qp_ms * 1e3, 2), "GB/s": round(qp_gbps, 1),
                              "frac_hbm": round(qp_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": qp_bytes}
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(name, wl, d, args.cpu_seconds, pow2)
    print(json.dumps(out), flush=True)
    return 0


def moe_main(args, wl) -> int:
    """One GPU's share of a MoE layer: group-quantize the expert-sorted rows,
    then the grouped block GEMM over the local experts (weights quantized
    beforehand, untimed)."""
    import numpy as np
    import torch

    import fp8_block_scaled_token_amd as fq

    _, off = wl.routing()
    M, N, K, E = int(off[-1]), wl.N, wl.K, wl.local_experts
    KB = K // 128
    x = wl.activations().cuda()
    offd = off.to(torch.int32).cuda()
    shard = wl.shard
    nbs = (N // shard) * math.ceil(shard / 128) if shard else math.ceil(N / 128)
    qw = torch.empty(E, N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(E, nbs, KB, dtype=torch.float32, device="cuda")
    for e in range(E):
        wd = wl.expert_weight(e, device="cuda")      # seeded per expert on the device
        if shard:
            nb = math.ceil(shard / 128)
            for i in range(N // shard):
                fq.fp8q_quant_weight_block(wd[i * shard:(i + 1) * shard], 128, 128, fq.SCALE_F32,
                                           qw[e, i * shard:(i + 1) * shard], sw[e, i * nb:(i + 1) * nb])
        else:
            fq.fp8q_quant_weight_block(wd, 128, 128, fq.SCALE_F32, qw[e], sw[e])
        del wd
    set_bytes = M * K * 3 + M * KB * 4 + M * N * 2
    nsets = max(2, min(8, math.ceil(MALL_DEFEAT_BYTES / set_bytes)))
    sets = [{"x": x.clone(), "q": torch.empty(M, K, dtype=torch.uint8, device="cuda"),
             "s": torch.empty(KB, M, dtype=torch.float32, device="cuda"),
             "y": torch.empty(M, N, dtype=torch.bfloat16, device="cuda")} for _ in range(nsets)]

    def quant(s):
        fq.fp8q_quant_act_group(s["x"], 128, fq.SCALE_F32, fq.COL_MAJOR, None, s["q"], s["s"])

    def gemm(s):
        fq.fp8q_gemm_grouped_blockscale(s["q"], s["s"], fq.COL_MAJOR, offd, qw, sw, s["y"], shard, fq.GRAN_BLOCK128)

    def step(i):
        quant(sets[i % nsets])
        gemm(sets[i % nsets])

    settle_clocks(step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    for i in range(args.steps):
        quant(sets[i % nsets])
        gemm(sets[i % nsets])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the grouped GEMM timed inside a second pass of the same steps (HIP
    # events around each launch, dispatch gap included) and back to back,
    # the tighter of the two for the roofline (as for the dense workloads);
    # the quantizer back to back
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        quant(sets[i % nsets])
        ev[i][0].record(stream)
        gemm(sets[i % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()

    def timed(fn, reps):
        return launch_ms(fn, sets, reps, stream, timing)

    timing = {}
    reps = max(args.steps, 2 * nsets)
    quant_ms = timed(quant, reps)
    gemm_b2b_ms = timed(gemm, reps)
    step_gemm_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    gemm_ms = min(step_gemm_ms, gemm_b2b_ms)
    flops = 2.0 * M * N * K
    g_bytes = E * N * K + M * K + 4 * M * KB + 4 * E * nbs * KB + 2 * M * N
    q_bytes = M * K * 3 + 4 * M * KB
    gemm_gbps = g_bytes / (gemm_ms * 1e-3) / 1e9
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    quant_gbps = q_bytes / (quant_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "N": N, "K": K, "experts": E, "tokens": wl.tokens,
                   "top_k": wl.top_k, "routed_experts": wl.n_experts, "shard": shard,
                   "scales": "group128 + 128x128 fp32 per expert", "rotating_buffer_sets": nsets},
        # weight streaming dominates: 2 flops per weight byte per routed row
        # (about 2 * 129 here) is below the chip's 625 flop/byte balance
        "roofline": {"bound": "hbm", "achieved": round(gemm_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gemm_gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(wl.name)},
        "gemm": {"us": round(gemm_ms * 1e3, 2), "TFLOP/s": round(gemm_tflops, 1),
                 "frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "GB/s": round(gemm_gbps, 1),
                 "algorithmic_bytes": g_bytes},
        "quant": {"kernel": "quant_group128", "us": round(quant_ms * 1e3, 2), "GB/s": round(quant_gbps, 1),
                  "frac_hbm": round(quant_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": q_bytes},
        "cpu_baseline": None,
    }
    out["gemm"]["us_in_step"] = round(step_gemm_ms * 1e3, 2)
    out["gemm"]["us_back_to_back"] = round(gemm_b2b_ms * 1e3, 2)
    out["kernel_timing"] = {"gemm": "in the steps" if step_gemm_ms <= gemm_b2b_ms else timing.get("kernel_timing"),
                            "quant": timing.get("kernel_timing")}
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = moe_cpu_baseline(wl, x.cpu(), off, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def moe_cpu_baseline(wl, x, off, target_s):
    """The oracle's group quantizer and grouped GEMM on the rows of the first
    experts (growing until about target_s of CPU time)."""
    import numpy as np
    from oracle import gemm as og
    from oracle import quant as oq
    off = off.numpy()
    xh = x.float().numpy()
    cache = {}

    def weight(e):
        if e not in cache:
            wh = wl.expert_weight(e, device="cuda").float().cpu().numpy()
            cache[e] = oq.quant_weight_block_sharded(wh, wl.shard) if wl.shard else oq.quant_weight_block(wh)
        return cache[e]

    n_exp = 1
    while True:
        for e in range(n_exp):
            weight(e)                                    # weight preparation is untimed
        rows = int(off[n_exp])
        t0 = time.perf_counter()
        qa, sa = oq.quant_group(xh[:rows])
        og.gemm_grouped_blockscale(qa, sa, lambda e: weight(e)[0], lambda e: weight(e)[1], off[:n_exp + 1],
                                   shard=wl.shard)
        t = time.perf_counter() - t0
        if t >= 0.5 * target_s or n_exp >= wl.local_experts or n_exp >= 8:
            break
        n_exp = min(wl.local_experts, 8, max(n_exp + 1, int(n_exp * 0.8 * target_s / max(t, 1e-3))))
    return {"value": 2.0 * rows * wl.N * wl.K / t / 1e12, "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"rows of the first {n_exp} of {wl.local_experts} experts ({rows} rows, {t:.1f} s; "
                      f"weights quantized beforehand, untimed)",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(name, wl, d, target_s, pow2=False):
    """Time the CPU oracle (as it stands) on a bounded row sample."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    from oracle import gemm as og
    from oracle import quant as oq

    M, N, K = wl.M, wl.N, wl.K
    xh = d["x"].float().numpy()
    wh = d["w"].float().numpy()
    if name == "mx":
        qw, sw = oq.quant_mx(wh)
    elif name == "pertensor":
        qw, sw = oq.quant_tensor(wh)
        sx = np.float32(np.float32(np.abs(xh).max()) / np.float32(448.0))
    elif pow2:
        qw, sw = oq.requant_weight_pow2(*oq.quant_weight_block(wh))
    else:
        qw, sw = oq.quant_weight_block(wh)
    gh = d["gamma"].float().numpy() if wl.norm else None
    hh = d["h"].float().numpy() if wl.residual else None

    def run(rows):
        xs = xh[:rows]
        if pow2 and wl.norm:
            r = oq.add_rmsnorm_quant(xs, np.zeros_like(xs), gh, d["eps"], pow2=True)
            og.gemm_blockscale(r["q"], r["s"], qw, sw)
        elif pow2:
            qa, sa = oq.quant_group_pow2(xs)
            og.gemm_blockscale(qa, sa, qw, sw)
        elif wl.residual:
            r = oq.add_rmsnorm_quant(xs, hh[:rows], gh, d["eps"])
            og.gemm_blockscale(r["q"], r["s"], qw, sw)
        elif wl.norm:
            r = oq.rmsnorm_quant(xs, gh, d["eps"])
            og.gemm_blockscale(r["q"], r["s"], qw, sw)
        elif name == "mx":
            qa, ea = oq.quant_mx(xs)
            og.gemm_mx(qa, ea, qw, sw)
        elif name == "pertensor":
            og.gemm_pertensor(oq.quant_static(xs, sx), sx, qw, sw)
        else:
            qa, sa = oq.quant_group(xs)
            og.gemm_blockscale(qa, sa, qw, sw)

    # grow the row sample until one run takes about target_s (or covers M)
    rows = min(M, 4)
    while True:
        t0 = time.perf_counter()
        run(rows)
        t = time.perf_counter() - t0
        if t >= 0.5 * target_s or rows >= M:
            break
        rows = int(min(M, max(2 * rows, rows * 0.8 * target_s / max(t, 1e-3))))
    tflops = 2.0 * rows * N * K / t / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": blas_threads or len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{rows} of {M} activation rows through the oracle's quantizer + GEMM "
                      f"({t:.1f} s; weight quantized beforehand, untimed)",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    sys.exit(main())
