#!/usr/bin/env python3
"""Benchmark of the fused row normalizations on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input, inputs resident in HBM:
  1. dual q/k head RMSNorm, bf16, q [4096,32,128] + k [4096,8,128], one launch
  2. RMSNorm bf16 [16384, 8192]
  3. LayerNorm bf16 [65536, 4096] (mean 3, 0.1% outliers x100), with bias

Metric: achieved HBM GB/s over the algorithmic bytes (read x once, write y
once, read the weights/bias once per launch) and rows/s.  Timing: whole steps
for at least 300 ms (the settle: per-kernel times drift down for the first
tens of ms of sustained load), W warm-up steps, then K steps bracketed by
synchronize and two HIP events on the stream the kernels run on (the step
time and ``value``).  Per kernel (``per_op``, and the roofline): the kernel
alone, launched back to back over input/output sets used in turn so every
launch is cold, two events around the launches.  K more steps with an event
after every launch give each kernel's time inside the step (``in_step``; the
events add about 12 us to a step).  The step order makes every input cold in
the caches: 1.6 GB of other traffic separates two reads of the same tensor,
more than the 256 MB MALL.

Prints ONE JSON line.  Extra legs (outside the timed region): the plain
copy kernel over the LayerNorm's bytes (practical ceiling), fused against
composed (ABBA), the dual launch with RoPE fused in, decode-sized calls
(eager and HIP-graph replay), RMSNorm with the SiLU-gate epilogue, and the
fp64 CPU oracle over full steps for about 10 s (``cpu_baseline``).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer_bf16_65536x4096_traffic.json")
KERNEL_SOURCES = ["fnorm_device.hpp", "fnorm_kernels.hpp", "fnorm_instances.hpp", "fnorm_api.hip"]


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks and empty lines, so
    that a comment edit does not count as a kernel change.  (String literals
    containing comment markers are not handled; the kernel sources have
    none.)"""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """Hash of the code (comments stripped) of the sources that define the
    bench's kernels and their launch configuration."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "transformer_row_normalization_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20,
                   help="untimed steps after the time-based settle")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-composed", action="store_true",
                   help="skip the fused-vs-composed ABBA comparison")
    p.add_argument("--ops", default="dual,rms,layer", help="subset of the step, for profiling")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on one GPU only; "
                          "rows shard across GPUs with no exchange, so the per-GPU kernel "
                          "is what one GPU measures"}))
        sys.exit(2)

    import torch

    import transformer_row_normalization_amd as trn
    from transformer_row_normalization_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops = args.ops.split(",")

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    log("[bench] generating inputs")
    wl_dual = inputs.dual_bf16_4096tok()
    wl_rms = inputs.rms_bf16_16384x8192()
    wl_ln = inputs.layer_bf16_65536x4096()
    d = {}
    for wl in (wl_dual, wl_rms, wl_ln):
        d[wl.name] = {k: v.to(dev) for k, v in wl.tensors.items() if torch.is_tensor(v)}
    dq, drms, dln = d[wl_dual.name], d[wl_rms.name], d[wl_ln.name]
    qy, ky = torch.empty_like(dq["q"]), torch.empty_like(dq["k"])
    y_rms = torch.empty_like(drms["x"])
    y_ln = torch.empty_like(dln["x"])

    def nbytes(*ts):
        return sum(t.numel() * t.element_size() for t in ts)

    plan = []   # (name, launch fn, algorithmic bytes, rows, kernel description)
    if "dual" in ops:
        plan.append(("dual_bf16_q131072_k32768_hd128",
                     lambda: trn.dual_head_rms_norm(dq["q"], dq["k"], dq["qw"], dq["kw"],
                                                    wl_dual.eps, q_out=qy, k_out=ky),
                     nbytes(dq["q"], dq["k"], dq["qw"], dq["kw"], qy, ky), wl_dual.rows,
                     trn.describe(trn.OP_DUAL, trn.BF16, 128)))
    if "rms" in ops:
        plan.append(("rms_bf16_16384x8192",
                     lambda: trn.rms_norm(drms["x"], drms["w"], wl_rms.eps, out=y_rms),
                     nbytes(drms["x"], drms["w"], y_rms), wl_rms.rows,
                     trn.describe(trn.OP_RMS, trn.BF16, 8192)))
    if "layer" in ops:
        plan.append(("layer_bf16_65536x4096",
                     lambda: trn.layer_norm(dln["x"], dln["w"], dln["b"], wl_ln.eps, out=y_ln),
                     nbytes(dln["x"], dln["w"], dln["b"], y_ln), wl_ln.rows,
                     trn.describe(trn.OP_LAYER, trn.BF16, 4096)))

    stream = torch.cuda.current_stream(dev)
    # Settle: whole steps for at least SETTLE_MS of sustained load before the
    # warm-up steps, so that the timed region does not depend on --warmup
    # (kernel times drift down over the first tens of ms of load)
    log(f"[bench] settle >= {SETTLE_MS} ms, then warmup {args.warmup} steps")
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
        for _ in range(10):
            for _, fn, _, _, _ in plan:
                fn()
        torch.cuda.synchronize()
        settle_steps += 10
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        for _, fn, _, _, _ in plan:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    # Timed region: exactly K steps, one event before and one after, so no
    # instrumentation sits between the kernels (an event record after every
    # kernel adds about 12 us to a step).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(K):
        for _, fn, _, _, _ in plan:
            fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K

    # Per-kernel region: K more steps with an event after every kernel, on
    # the stream the kernels run on; per-kernel durations and the roofline
    # come from here.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)] for _ in range(K)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {K} instrumented steps (per-kernel events)")
    torch.cuda.synchronize()
    s0.record(stream)
    for s in range(K):
        evs[s][0].record(stream)
        for i, (_, fn, _, _, _) in enumerate(plan):
            fn()
            evs[s][i + 1].record(stream)
    s1.record(stream)
    torch.cuda.synchronize()
    ms_per_step_instrumented = s0.elapsed_time(s1) / K

    per_op = {}
    for i, (name, _, b, rows, kname) in enumerate(plan):
        durs = sorted(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(K))
        avg = sum(durs) / K
        per_op[name] = {"kernel": kname, "bytes": b, "rows": rows,
                        "in_step": {"avg_ms": round(avg, 5), "min_ms": round(durs[0], 5),
                                    "median_ms": round(durs[K // 2], 5),
                                    "gbs": round(b / (avg * 1e-3) / 1e9, 1),
                                    "frac_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                    "note": "an event record after every kernel of the step; "
                                            "includes part of the events' cost and the write-back "
                                            "of lines the previous kernel left dirty"}}

    # Each kernel alone: launches back to back on the step's stream, with
    # enough input/output sets used in turn that every launch reads data the
    # previous ones evicted from the 256 MB MALL and writes lines no earlier
    # launch left dirty; two events around N launches give the average launch
    # duration with no instrumentation between launches (each set's call
    # prepared once, see standalone_arms).  The roofline uses this figure.
    for name, alone in standalone_arms(torch, trn, plan, dq, drms, dln, wl_dual, wl_rms,
                                       wl_ln).items():
        n_alone = max(K, 30)
        for _ in range(2 * alone["sets"]):
            alone["fn"]()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(n_alone):
            alone["fn"]()
        a1.record(stream)
        torch.cuda.synchronize()
        avg = a0.elapsed_time(a1) / n_alone
        if ":" in name:   # an alternative policy of a step kernel, reported beside it
            base, tag = name.split(":")
            op = per_op[base]
            op[f"alone_{tag}_stores"] = {
                "kernel": alone["kernel"], "avg_ms": round(avg, 5),
                "gbs": round(op["bytes"] / (avg * 1e-3) / 1e9, 1),
                "frac_peak": round(op["bytes"] / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "note": "not the default: inside the step this policy made the step slower "
                        "(ordinary stores leave the output in the MALL and their write-back "
                        "overlaps the next kernel)"}
            log(f"[bench] {name}: {op[f'alone_{tag}_stores']}")
            continue
        op = per_op[name]
        op.update({"avg_ms": round(avg, 5), "launches": n_alone, "buffer_sets": alone["sets"],
                   "gbs": round(op["bytes"] / (avg * 1e-3) / 1e9, 1),
                   "frac_peak": round(op["bytes"] / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "rows_per_s": round(op["rows"] / (avg * 1e-3), 1)})
        log(f"[bench] {name}: {op}")
    torch.cuda.empty_cache()
    step_bytes = sum(p[2] for p in plan)
    step_rows = sum(p[3] for p in plan)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # practical ceiling: the 16-byte copy kernel moving the same bytes as the
    # LayerNorm (the dominant kernel) and as the dual launch (small enough
    # that the launch's ramp-up and tail show).  Consecutive copies use
    # different slices of the 512 MiB LayerNorm buffers, so that, like the
    # step's kernels, each one reads cold data (a slice read again while
    # still in the 256 MB MALL would time the cache, not HBM).
    def copy_ceiling(nbytes_each_way):
        src_all = dln["x"].view(-1).view(torch.uint8)
        dst_all = y_ln.view(-1).view(torch.uint8)
        slices = max(1, src_all.numel() // nbytes_each_way)
        pairs = [(src_all[i * nbytes_each_way:(i + 1) * nbytes_each_way],
                  dst_all[i * nbytes_each_way:(i + 1) * nbytes_each_way]) for i in range(slices)]
        reps = 20

        def timed(copy):
            for i in range(3):
                copy(*pairs[i % slices])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                copy(*pairs[(i + 3) % slices])
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        cms = timed(trn.bench_copy)
        # the runtime's own device-to-device copy (torch's copy_ of two
        # contiguous byte tensors is a hipMemcpyAsync)
        mms = timed(lambda s_, d_: d_.copy_(s_))
        return {"kernel": "copy16 (fnorm_bench_copy)", "bytes": 2 * nbytes_each_way,
                "avg_ms": round(cms, 5), "distinct_slices": slices,
                "gbs": round(2 * nbytes_each_way / (cms * 1e-3) / 1e9, 1),
                "d2d_memcpy": {"avg_ms": round(mms, 5),
                               "gbs": round(2 * nbytes_each_way / (mms * 1e-3) / 1e9, 1)}}

    ceiling = None
    if "layer" in ops:
        ceiling = copy_ceiling(dln["x"].numel() * dln["x"].element_size())
        if "dual" in ops:
            qk = nbytes(dq["q"], dq["k"])
            ceiling["at_dual_bytes"] = copy_ceiling(qk - qk % 16)
        log(f"[bench] copy ceiling: {ceiling}")
        # each kernel against the copy kernel at (about) its own size
        for name, op in per_op.items():
            ref = ceiling.get("at_dual_bytes", ceiling) if name.startswith("dual") else ceiling
            op["frac_copy"] = round(op["gbs"] / ref["gbs"], 4)

    dominant = max(per_op, key=lambda k: per_op[k]["avg_ms"])
    dom = per_op[dominant]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == dominant:
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(dom["bytes"] / (dom["avg_ms"] * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dom["bytes"] / (dom["avg_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "traffic": traffic, "kernel": dominant,
                "duration": "average launch duration of the kernel alone (per_op)"}

    composed = None
    rope = None
    decode = None
    gated = None
    if not args.no_composed and len(plan) == 3:
        composed = fused_vs_composed(trn, inputs, dev, stream, d, wl_rms, wl_ln, log)
        rope = dual_rope_leg(trn, dq, qy, ky, wl_dual.eps, stream, log)
        decode = decode_leg(trn, dev, stream, log)
        gated = gated_leg(trn, inputs, dev, stream, log)

    cpu = None
    if not args.no_cpu_baseline and len(plan) == 3:
        cpu = cpu_baseline(wl_dual, wl_rms, wl_ln, log)

    # the device as the runtime reports it.  The bus moves bus_bits / 8
    # bytes per transfer; HBM3E makes four transfers per reported memory
    # clock (8 Gb/s per pin at 2.0 GHz), so the runtime's figures give
    # clock * 4 * bus_bits / 8 as peak (the roofline uses the published
    # 8 TB/s)
    props = torch.cuda.get_device_properties(dev)
    mem = trn.device_memory()
    per_clock = mem["memory_clock_khz"] * 1e3 * mem["memory_bus_bits"] / 8 / 1e9
    device = {"name": props.name, "arch": props.gcnArchName, **mem,
              "total_memory_gib": round(props.total_memory / 2**30, 1),
              "gbs_per_transfer_per_clock": round(per_clock, 1),
              "props_peak_gbs": round(4 * per_clock, 1),
              "published_peak_gbs": PEAK_HBM_GBS}
    log(f"[bench] device: {device}")

    out = {"metric": "achieved HBM GB/s (% of peak) and rows/sec for fused RMSNorm/LayerNorm",
           "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic (seeded, shapes and distributions of the workloads)",
           "config": {"workload": "step = " + " + ".join(p[0] for p in plan),
                      "io_dtype": "bf16", "accumulate": "f32",
                      "rows_per_step": step_rows, "bytes_per_step": step_bytes,
                      "rows_per_s": round(step_rows / (ms_per_step * 1e-3), 1),
                      "frac_peak_hbm": round(value / PEAK_HBM_GBS, 4),
                      "parallelism": "rows across workgroups (1 GPU)",
                      "layer_outliers": int(wl_ln.tensors["outliers"])},
           "timing": {"value": f"{K} steps between two events on the launch stream, after "
                               f"a {settle_ms:.0f} ms settle ({settle_steps} steps) and "
                               f"{args.warmup} warm-up steps",
                      "per_op": "each kernel alone: launches back to back over input/output "
                                "sets used in turn (cold), each set's call prepared once "
                                "(trn.prepare: relaunched through the C entry point), two "
                                "events around them",
                      "per_op_in_step": f"{K} further steps with an event after every kernel",
                      "settle_ms": round(settle_ms, 1), "settle_steps": settle_steps,
                      "ms_per_step_instrumented": round(ms_per_step_instrumented, 5)},
           "device": device, "per_op": per_op, "copy_ceiling": ceiling,
           "roofline": roofline, "cpu_baseline": cpu,
           "small_configs": small_configs(composed, inputs),
           "fused_vs_composed": composed,
           "dual_rope": rope, "decode": decode, "rms_swiglu": gated,
           "wall_s_timed_region": round(wall, 4)}
    print(json.dumps(out), flush=True)


SETTLE_MS = 300.0


def standalone_arms(torch, trn, plan, dq, drms, dln, wl_dual, wl_rms, wl_ln):
    """Per kernel of the step: a launch function that uses its own input/output
    sets in turn, as many as make each launch's footprint, summed over the
    sets, exceed 512 MiB (so no launch finds its rows in the MALL).  Each set's
    call is bound once with the binding's `prepare` (validated once, then
    relaunched through the C entry point), so that the Python checks of a
    call (~6 us) do not leave the GPU waiting between short launches."""
    out = {}
    names = [p[0] for p in plan]

    def sets_for(nbytes):
        return max(2, -(-(512 << 20) // nbytes) + 1)

    def rotate(launches):
        turn = [0]

        def fn():
            launches[turn[0]]()
            turn[0] = (turn[0] + 1) % len(launches)
        return fn

    for name in names:
        if name.startswith("dual"):
            n = sets_for(2 * (dq["q"].numel() + dq["k"].numel()) * 2)
            sets = [(dq["q"].clone(), dq["k"].clone(), torch.empty_like(dq["q"]),
                     torch.empty_like(dq["k"])) for _ in range(n)]
            calls = [trn.prepare(trn.dual_head_rms_norm, q, k, dq["qw"], dq["kw"], wl_dual.eps,
                                 q_out=a, k_out=b)[0] for q, k, a, b in sets]
        elif name.startswith("rms"):
            n = sets_for(2 * drms["x"].numel() * 2)
            sets = [(drms["x"] if i == 0 else drms["x"].clone(), torch.empty_like(drms["x"]))
                    for i in range(n)]
            calls = [trn.prepare(trn.rms_norm, x, drms["w"], wl_rms.eps, out=y)[0]
                     for x, y in sets]
            # the same shape with non-temporal stores, when the default keeps
            # ordinary ones (the store policy is a trade-off: an ordinary
            # store leaves the output in the MALL for its consumer, and its
            # write-back overlaps the next kernel; alone, non-temporal stores
            # are faster)
            width = drms["x"].shape[-1]
            default = trn.describe(trn.OP_RMS, trn.BF16, width)
            if ".ntld." in default:
                want = default.replace(".ntld.", ".nt.")
                for v in range(trn.variant_count(trn.OP_RMS, trn.BF16, width)):
                    if trn.describe(trn.OP_RMS, trn.BF16, width, variant=v) == want:
                        alt = [trn.prepare(trn.rms_norm, x, drms["w"], wl_rms.eps, out=y,
                                           variant=v)[0] for x, y in sets]
                        out[name + ":nt"] = {"fn": rotate(alt), "sets": n, "kernel": want,
                                             "keep": sets}
                        break
        else:
            n = sets_for(2 * dln["x"].numel() * 2)
            sets = [(dln["x"] if i == 0 else dln["x"].clone(), torch.empty_like(dln["x"]))
                    for i in range(n)]
            calls = [trn.prepare(trn.layer_norm, x, dln["w"], dln["b"], wl_ln.eps, out=y)[0]
                     for x, y in sets]
        out[name] = {"fn": rotate(calls), "sets": n, "keep": sets}
    return {k: out[k] for k in sorted(out, key=lambda k: (k.split(":")[0] not in names, k))}


def small_configs(composed, inputs):
    """The two page-shaped workloads (the notebook's Part 1 RMSNorm input and
    the kernel_micro_ab LayerNorm shape) in the metric's units, from the cold
    arm of the fused-vs-composed leg: GB/s over the algorithmic bytes
    (x in, y out, weights), rows/s and the fraction of 8 TB/s.  At 4-6 MB a
    call is bound by its launch and ramp, not by HBM."""
    if not composed:
        return None
    out = {}
    for key, wl in (("rms_f32_4x128x1024_iota", inputs.rms_f32_512x1024("iota")),
                    ("layer_f32_1x1024x768", inputs.layer_f32_1024x768())):
        rec = composed.get(key, {}).get("cold")
        if not rec:
            continue
        t = wl.tensors
        nbytes = 2 * t["x"].numel() * 4 + t["w"].numel() * 4 + (
            t["b"].numel() * 4 if "b" in t else 0)
        rows = t["x"].numel() // t["x"].shape[-1]
        us = rec["fused"]["min_us"]
        out[key] = {"us_min": us, "us_mean": rec["fused"]["mean_us"], "bytes": nbytes,
                    "rows": rows, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "rows_per_s": round(rows / (us * 1e-6), 1),
                    "frac_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "bound": "launch (4-6 MB per call)",
                    "cache": "cold: a 512 MiB copy evicts the MALL before every timed call"}
    return out


def fused_vs_composed(trn, inputs, dev, stream, d, wl_rms, wl_ln, log):
    """The pages' own experiment on this GPU: the fused kernel against the
    same formula run one primitive per launch (6 launches for RMSNorm, 9 for
    LayerNorm with bias), interleaved ABBA (the arm order flips every rep so
    a drift cannot favour one arm), 30 reps, per-call time on the stream,
    minimum and mean kept.  Shapes: the notebook's Part 1 RMSNorm input, the
    kernel_micro_ab LayerNorm input, and the two large workloads."""
    import torch

    reps = 30
    small_r = inputs.rms_f32_512x1024("iota")
    small_l = inputs.layer_f32_1024x768()
    cases = []
    for name, wl, op in (("rms_f32_4x128x1024_iota", small_r, "rms"),
                         ("layer_f32_1x1024x768", small_l, "layer"),
                         ("rms_bf16_16384x8192", wl_rms, "rms"),
                         ("layer_bf16_65536x4096", wl_ln, "layer")):
        t = d.get(wl.name) or {k: v.to(dev) for k, v in wl.tensors.items() if torch.is_tensor(v)}
        fused, comp, nbytes = _arms(trn, torch, op, t, wl.eps)
        cases.append((name, fused, comp, nbytes))
    # a 512 MiB copy between two scratch buffers evicts the 256 MB MALL
    flush_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)

    def flush():
        trn.bench_copy(flush_src, flush_dst)

    def abba(fused, comp, nbytes, before=None):
        for f in (fused, comp, fused, comp):
            f()
        torch.cuda.synchronize()
        times = {"fused": [], "composed": []}
        for r in range(reps):
            arms = (("fused", fused), ("composed", comp))
            if r % 2:
                arms = arms[::-1]
            for arm, f in arms:
                if before:
                    before()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                f()
                e1.record(stream)
                torch.cuda.synchronize()
                times[arm].append(e0.elapsed_time(e1) * 1e3)
        rec = {arm: {"min_us": round(min(v), 2), "mean_us": round(sum(v) / len(v), 2)}
               for arm, v in times.items()}
        rec["speedup_min"] = round(rec["composed"]["min_us"] / rec["fused"]["min_us"], 2)
        rec["fused_gbs"] = round(nbytes / (rec["fused"]["min_us"] * 1e-6) / 1e9, 1)
        return rec

    out = {}
    for name, fused, comp, nbytes in cases:
        if nbytes < (64 << 20):
            # fits in the MALL: repeated calls time it warm; cold calls
            # follow a flush (outside the timed region)
            rec = abba(fused, comp, nbytes)
            rec["cache"] = "warm: inputs and outputs stay in the 256 MB MALL between calls"
            rec["cold"] = abba(fused, comp, nbytes, before=flush)
            rec["cold"]["cache"] = "cold: a 512 MiB copy evicts the MALL before every timed call"
        else:
            rec = abba(fused, comp, nbytes)
            rec["cache"] = "cold: the tensors exceed the 256 MB MALL"
        out[name] = rec
        log(f"[bench] fused vs composed {name}: {rec}")
        torch.cuda.empty_cache()
    del flush_src, flush_dst
    return out


def _abba_back_to_back(torch, stream, arms, reps=12, calls=20):
    """Median and minimum per-launch time (us) of each arm: `calls` launches
    back to back between two events on the stream, arms in ABBA order over
    `reps` repetitions."""
    for f in arms.values():
        for _ in range(calls):
            f()
    torch.cuda.synchronize()
    times = {k: [] for k in arms}
    for r in range(reps):
        for k in (list(arms) if r % 2 == 0 else list(arms)[::-1]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(calls):
                arms[k]()
            e1.record(stream)
            torch.cuda.synchronize()
            times[k].append(e0.elapsed_time(e1) * 1e3 / calls)
    out = {}
    for k, v in times.items():
        v = sorted(v)
        out[k] = {"median_us": round((v[(reps - 1) // 2] + v[reps // 2]) / 2, 2),
                  "min_us": round(v[0], 2)}
    return out


def _rotating(calls):
    turn = [0]

    def fn():
        calls[turn[0]]()
        turn[0] = (turn[0] + 1) % len(calls)
    return fn


def dual_rope_leg(trn, dq, qy, ky, eps, stream, log):
    """The dual workload with the rotary embedding fused into the same launch
    (positions 0..4095, base 10000, split-half) against the plain dual norm
    and the copy kernel over the same bytes.  Cold: 8 copies of the inputs
    (672 MB) are used in turn, so no call finds its rows in the 256 MB MALL.
    Each set's call is prepared once; 20 launches back to back between two
    events, ABBA over 12 reps, medians.  The rotation adds no HBM traffic."""
    import torch

    sets = [(dq["q"].clone(), dq["k"].clone(), torch.empty_like(qy), torch.empty_like(ky))
            for _ in range(8)]
    flat = [(torch.cat([q.reshape(-1), k.reshape(-1)]),
             torch.empty(q.numel() + k.numel(), dtype=q.dtype, device=q.device))
            for q, k, _, _ in sets]
    arms = {
        "dual": _rotating([trn.prepare(trn.dual_head_rms_norm, q, k, dq["qw"], dq["kw"], eps,
                                       q_out=a, k_out=b)[0] for q, k, a, b in sets]),
        "dual_rope": _rotating([trn.prepare(trn.dual_head_rms_rope, q, k, dq["qw"], dq["kw"],
                                            eps, q_out=a, k_out=b)[0] for q, k, a, b in sets]),
        "copy": _rotating([(lambda s_=s_, d_=d_: trn.bench_copy(s_, d_)) for s_, d_ in flat])}
    out = _abba_back_to_back(torch, stream, arms)
    nbytes = 2 * (dq["q"].numel() + dq["k"].numel()) * 2
    for k, rec in out.items():
        gbs = nbytes / (rec["median_us"] * 1e-6) / 1e9
        rec.update({"gbs_median": round(gbs, 1), "frac_peak": round(gbs / PEAK_HBM_GBS, 4)})
    out["dual_rope"]["frac_copy"] = round(out["copy"]["median_us"] /
                                          out["dual_rope"]["median_us"], 4)
    out["kernel"] = trn.describe_rope(trn.BF16, 128, 128, False)
    out["bytes"] = nbytes
    out["cache"] = "cold: 8 input copies used in turn; prepared calls back to back"
    del sets, flat
    log(f"[bench] dual + rope: {out}")
    return out


def gated_leg(trn, inputs, dev, stream, log):
    """RMSNorm with the SiLU-gate epilogue at the gated-delta output-norm
    shape (4096 tokens x 32 heads x 128, bf16) against the plain RMSNorm of
    the same x and the copy kernel over each one's bytes: 8 input copies used
    in turn (cold), prepared calls, 20
    launches back to back between two events, ABBA over 12 reps.  The fused
    epilogue adds the gate read (6 bytes per element against 4); run as a
    separate pass it would re-read y and the gate and write y again."""
    import torch

    wl = inputs.rms_swiglu_bf16_4096tok()
    x0, g0, w = (wl.tensors[k].to(dev) for k in ("x", "g", "w"))
    sets = [(x0.clone(), g0.clone(), torch.empty_like(x0)) for _ in range(8)]
    n = x0.numel()
    # the copy kernel over the same total bytes: n elements in and out for the
    # plain norm, 1.5 n for the gated one (x and g in, y out)
    flat = {m: [(torch.empty(m, dtype=x0.dtype, device=dev), torch.empty(m, dtype=x0.dtype, device=dev))
                for _ in range(8)] for m in (n, 3 * n // 2)}
    arms = {"rms": _rotating([trn.prepare(trn.rms_norm, x, w, wl.eps, out=y)[0]
                              for x, _, y in sets]),
            "rms_swiglu": _rotating([trn.prepare(trn.rms_norm_swiglu, x, g, w, wl.eps, out=y)[0]
                                     for x, g, y in sets]),
            "copy_rms_bytes": _rotating([(lambda s_=s_, d_=d_: trn.bench_copy(s_, d_))
                                         for s_, d_ in flat[n]]),
            "copy_rms_swiglu_bytes": _rotating([(lambda s_=s_, d_=d_: trn.bench_copy(s_, d_))
                                                for s_, d_ in flat[3 * n // 2]])}
    nbytes = {"rms": 2 * n * 2, "rms_swiglu": 3 * n * 2, "copy_rms_bytes": 2 * n * 2,
              "copy_rms_swiglu_bytes": 3 * n * 2}
    out = _abba_back_to_back(torch, stream, arms)
    for k, rec in out.items():
        gbs = nbytes[k] / (rec["median_us"] * 1e-6) / 1e9
        rec.update({"bytes": nbytes[k], "gbs_median": round(gbs, 1),
                    "frac_peak": round(gbs / PEAK_HBM_GBS, 4)})
    for k in ("rms", "rms_swiglu"):
        out[k]["frac_copy"] = round(out[f"copy_{k}_bytes"]["median_us"] / out[k]["median_us"], 4)
    out["shape"] = "x, g [4096, 32, 128] bf16 (131072 rows of 128)"
    out["kernel"] = trn.describe(trn.OP_RMS_SWIGLU, trn.BF16, 128)
    out["cache"] = "cold: 8 input copies used in turn; prepared calls back to back"
    del sets, flat
    log(f"[bench] gated output norm: {out}")
    return out


def decode_leg(trn, dev, stream, log):
    """Decode-sized calls, where launches dominate: one decode step of the
    dual workload's head layout (32 query heads, 8 key heads, head_dim 128,
    bf16) at 1, 8 and 64 tokens.  Arms per layer: two single RMSNorm
    launches (q, then k), the one dual launch, and the dual launch with RoPE
    (position 1000 + token).  Timed two ways, ABBA over the arms:
      eager  - 200 back-to-back calls between two events: what a host loop
               sustains, launch submission included ("dual_c_abi" calls the
               C entry point directly with prepared arguments, leaving out
               the Python binding's checks; "dual_prepared" is the binding's
               own prepared call, `prepare`);
      graph  - one HIP graph holding 64 calls, replayed 10 times: device
               time per call with the host out of the loop."""
    import torch

    g = torch.Generator().manual_seed(5)
    qh, kh, hd = 32, 8, 128
    out = {}
    for tokens in (1, 8, 64):
        q = torch.randn(tokens, qh, hd, generator=g).to(torch.bfloat16).to(dev)
        k = torch.randn(tokens, kh, hd, generator=g).to(torch.bfloat16).to(dev)
        qw = (1 + 0.1 * torch.randn(hd, generator=g)).to(torch.bfloat16).to(dev)
        kw = (1 + 0.1 * torch.randn(hd, generator=g)).to(torch.bfloat16).to(dev)
        qy, ky = torch.empty_like(q), torch.empty_like(k)
        # the C entry point called directly with prepared arguments: the
        # library's own host cost per launch, without the binding's checks
        import ctypes
        c_args = tuple(ctypes.c_void_p(t.data_ptr()) for t in (q, k, qw, kw, qy, ky)) + (
            tokens * qh, tokens * kh, hd, ctypes.c_float(1e-6), trn.BF16,
            ctypes.c_void_p(stream.cuda_stream))
        c_dual = trn.lib().fnorm_dual_head_rms
        prepared, _ = trn.prepare(trn.dual_head_rms_norm, q, k, qw, kw, 1e-6, q_out=qy, k_out=ky)
        arms = {
            "dual_c_abi": lambda: c_dual(*c_args),
            "dual_prepared": prepared,
            "two_rms": lambda: (trn.rms_norm(q, qw, 1e-6, out=qy), trn.rms_norm(k, kw, 1e-6, out=ky)),
            "dual": lambda: trn.dual_head_rms_norm(q, k, qw, kw, 1e-6, q_out=qy, k_out=ky),
            "dual_rope": lambda: trn.dual_head_rms_rope(q, k, qw, kw, 1e-6, offset=1000,
                                                        q_out=qy, k_out=ky)}
        graphs = {}
        for name, f in arms.items():
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            if name in ("dual_c_abi", "dual_prepared"):
                continue      # their bound stream is not the capture stream
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(64):
                    f()
            graphs[name] = gr
        times = {n: {"eager": [], "graph": []} for n in arms}
        for r in range(6):
            order = list(arms) if r % 2 == 0 else list(arms)[::-1]
            for name in order:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(200):
                    arms[name]()
                e1.record(stream)
                torch.cuda.synchronize()
                times[name]["eager"].append(e0.elapsed_time(e1) * 1e3 / 200)
                if name not in graphs:
                    continue
                graphs[name].replay()
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(10):
                    graphs[name].replay()
                e1.record(stream)
                torch.cuda.synchronize()
                times[name]["graph"].append(e0.elapsed_time(e1) * 1e3 / 640)
        rec = {n: {m: round(min(v), 2) for m, v in t.items() if v} for n, t in times.items()}
        rec["unit"] = "us per call (min over 6 ABBA reps)"
        out[f"tokens_{tokens}"] = rec
        log(f"[bench] decode tokens={tokens}: {rec}")
        del graphs
    return out


def _arms(trn, torch, op, t, eps):
    """(fused call, composed call, algorithmic bytes) bound to these tensors."""
    x, w, b = t["x"], t["w"], t.get("b")
    y = torch.empty_like(x)
    ws = trn.composed_workspace(trn.OP_RMS if op == "rms" else trn.OP_LAYER, x)
    nbytes = 2 * x.numel() * x.element_size()
    if op == "rms":
        return (lambda: trn.rms_norm(x, w, eps, out=y),
                lambda: trn.rms_norm_composed(x, w, eps, out=y, workspace=ws), nbytes)
    return (lambda: trn.layer_norm(x, w, b, eps, out=y),
            lambda: trn.layer_norm_composed(x, w, b, eps, out=y, workspace=ws), nbytes)


def cpu_baseline(wl_dual, wl_rms, wl_ln, log):
    """The fp64 oracle, as it stands, over one full step of the same inputs
    (row chunks, single thread); reported in the metric's unit over the same
    algorithmic bytes."""
    import oracle
    from tests import helpers

    o = oracle.default()
    log("[bench] cpu baseline (oracle, 1 thread, full steps for >= 10 s)")
    t = wl_dual.tensors
    arr = {k: helpers.to_oracle_array(t[k]) for k in ("q", "k", "qw", "kw")}
    big = []
    for wl, op in ((wl_rms, "rms"), (wl_ln, "layer")):
        b = helpers.to_oracle_array(wl.tensors["b"]) if "b" in wl.tensors else None
        big.append((op, helpers.to_oracle_array(wl.tensors["x"]),
                    helpers.to_oracle_array(wl.tensors["w"]), b, wl.eps))
    step_bytes = sum(v.nbytes for v in arr.values()) + arr["q"].nbytes + arr["k"].nbytes
    step_bytes += sum(2 * x.nbytes + w.nbytes + (b.nbytes if b is not None else 0)
                      for _, x, w, b, _ in big)
    steps = 0
    t0 = time.perf_counter()
    while True:
        o.dual_head_rms(arr["q"], arr["k"], arr["qw"], arr["kw"], wl_dual.eps)
        for op, x, w, b, eps in big:
            for r0 in range(0, x.shape[0], 2048):
                if op == "rms":
                    o.rms(x[r0:r0 + 2048], w, eps)
                else:
                    o.layer(x[r0:r0 + 2048], w, b, eps)
        steps += 1
        if time.perf_counter() - t0 >= 10.0:
            break
    dt = time.perf_counter() - t0
    return {"value": round(steps * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 3), "steps": steps,
            "sample": f"{steps} full steps (all rows of the three workloads) through the fp64 C "
                      "oracle, single thread, outputs in 2048-row chunks; same algorithmic bytes",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
