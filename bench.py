"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-secondary]
                    [--no-cpu-baseline]

One step = one training-mode forward of one DeepSeekMoE layer over one batch of synthetic
tokens: route -> permute -> [fp8 quantisation of x] -> gate/up grouped GEMM + SwiGLU ->
down grouped GEMMs -> combine -> bias update.  Inputs and weights are resident in HBM
before the timed region.  The headline workload is the DeepSeek-V3-shaped bf16 layer at
T = 4096 tokens (d = 7168, 256 routed + 1 shared SwiGLU experts of width 2048, top-8);
the fp8 layer at T = 16384, the group-limited bf16 layer at T = 8192 and the decode-shaped
fp8 run (T = 256, Zipf-skewed bias, 100 steps of the bias update) are reported in the same
line under "secondary", with the fp8 layer at T = 16384 also run with power-of-two (E8M0)
tile scales.  A workload name ending in "_e8m0" selects those scales for the main run.

Prints ONE JSON line.  Weights are random (no checkpoint); inputs are seeded synthetic data.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="v3_bf16_T4096")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--decode-steps", type=int, default=None)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first copy 1 GiB device-to-device twice (the reference dispatch for HBM counters)")
    p.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of a --calibrate-copy bench "
                        "into profiles/traffic_<kernel>_<workload>.json, then exit")
    return p.parse_args()


class KernelTimer:
    """HIP events around one launch on the stream it runs on; averages over the timed steps."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def wrap(self, fn, *a, **kw):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record(t.cuda.current_stream())
        r = fn(*a, **kw)
        e.record(t.cuda.current_stream())
        self.pairs.append((s, e))
        return r

    def mean_ms(self):
        if not self.pairs:
            return None
        return sum(s.elapsed_time(e) for s, e in self.pairs) / len(self.pairs)


def run_layer_steps(torch, M, layer, xs, steps, warmup, timer_gate_up, gamma, update_bias=True):
    """Warm up, then time `steps` forwards (events on the current stream)."""
    L = M._lib
    orig = L.moe_grouped_gemm
    state = {"timing": False}

    def gg(*a, **kw):
        if state["timing"] and kw.get("swiglu"):
            return timer_gate_up.wrap(orig, *a, **kw)
        return orig(*a, **kw)

    import sparse_moe_layer_sigmoid_amd.layer as layer_mod
    layer_mod.L.moe_grouped_gemm = gg
    try:
        for i in range(warmup):
            layer.forward(xs[i % len(xs)], update_bias=update_bias, gamma=gamma)
        torch.cuda.synchronize()
        state["timing"] = True
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            layer.forward(xs[i % len(xs)], update_bias=update_bias, gamma=gamma)
        end.record()
        torch.cuda.synchronize()
        state["timing"] = False
        return start.elapsed_time(end) / steps
    finally:
        layer_mod.L.moe_grouped_gemm = orig


def gate_up_bytes(cfg, counts_np, fp8: bool, scale_bytes: int = 4):
    """Algorithmic HBM bytes of one gate/up launch: the W13 of every expert with at least one
    row (plus the shared one) read once, each gathered input row read once, h written once
    (fp8: with their scales, scale_bytes each)."""
    esz = 1 if fp8 else 2
    sb = scale_bytes if fp8 else 0
    active = int((counts_np > 0).sum()) + 1
    w = active * 2 * cfg.inter * cfg.d * esz + active * (2 * cfg.inter // 128) * (cfg.d // 128) * sb
    rows = cfg.rows
    a = rows * cfg.d * esz + rows * (cfg.d // 128) * sb
    h = rows * cfg.inter * esz + rows * (cfg.inter // 128) * sb
    return w + a + h


def step_bytes(cfg, counts_np, fp8: bool):
    """Algorithmic bytes of one whole-layer step (weights of active experts + router once,
    x in, out written): the decode-shaped run's GB/s numerator."""
    esz = 1 if fp8 else 2
    active = int((counts_np > 0).sum()) + 1
    w = active * 3 * cfg.inter * cfg.d * esz
    if fp8:
        w += active * ((2 * cfg.inter // 128) * (cfg.d // 128) + (cfg.d // 128) * (cfg.inter // 128)) * 4
    return w + cfg.n_experts * cfg.d * 2 + 2 * cfg.T * cfg.d * 2


def kernel_src_sha():
    h = hashlib.sha256()
    for f in ("gemm.hip", "device_common.h"):
        with open(os.path.join(ROOT, "sparse_moe_layer_sigmoid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_tag):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they were taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_src_sha():
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def _pmc_rows(d, counter):
    """(kernel name, value) per dispatch of `counter` from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return [(k[1], v) for k, v in sorted(out.items(), key=lambda kv: int(kv[0][0]))]


def ingest_pmc(fetch_dir, write_dir, workload):
    """HBM bytes per launch of the gate/up kernel from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that maps the same counter on a 1 GiB device copy
    to 1 GiB."""
    # template arguments <..., input kind (0 bf16, 1 E4M3 + f32 scales, 2 E4M3 + E8M0), SwiGLU, output>
    kind = 2 if workload.endswith("_e8m0") else (1 if "fp8" in workload else 0)
    want = f"{kind}, true, {2 if kind else 0}>"
    rec = {"workload": workload, "kernel_src_sha": kernel_src_sha(), "copy_bytes": COPY_BYTES}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        copies = [v for n, v in rows if "copyBuffer" in n and v * 1024 > COPY_BYTES / 4]
        gemm = [v for n, v in rows if "grouped_gemm_kernel" in n and want in n]
        if not copies or not gemm:
            raise SystemExit(f"{counter}: no calibration copy or no gate/up dispatch in {d}")
        factor = COPY_BYTES / (sum(copies) / len(copies) * 1024)
        kib = sum(gemm) / len(gemm)
        rec[counter.lower()] = {"kib_per_dispatch": round(kib, 1), "copy_factor": round(factor, 4),
                                "bytes_per_launch": int(kib * 1024 * factor), "dispatches": len(gemm)}
    rec["bytes_per_launch"] = rec["fetch_size"]["bytes_per_launch"] + rec["write_size"]["bytes_per_launch"]
    path = os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(cfg, wr_cpu, bias_cpu, W13_cpu, W2_cpu, budget_s=10.0, max_steps=8):
    """The CPU oracle, untuned, on whole steps of the workload: per step, fp64 routing of all
    T tokens of a fresh batch, the permutation, the SwiGLU FFN of every expert (the shared
    one included) on the rows routed to it, the combine and the bias update; steps are
    repeated until `budget_s` seconds of oracle compute have run.  The fp64 copies of each
    expert's bf16 weights are made outside the timed region."""
    import numpy as np
    import torch

    from oracle import moe_oracle as O
    from sparse_moe_layer_sigmoid_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    wr64 = wr_cpu.double().numpy()
    timed, steps = 0.0, 0
    while steps < max_steps and (steps == 0 or timed < budget_s):
        x64 = I.gen_x(cfg, step=None if steps == 0 else steps).to(torch.bfloat16).double().numpy()
        t0 = time.perf_counter()
        r = O.route(x64, wr64, bias_cpu.numpy(), cfg.top_k, cfg.n_group, cfg.topk_group)
        offsets, sorted_token, pair_pos = O.permute(r["idx"], cfg.n_experts, 1)
        y_routed = np.empty((cfg.T * cfg.top_k, cfg.d))
        y_shared = None
        timed += time.perf_counter() - t0
        for e in range(cfg.n_experts + 1):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi == lo:
                continue
            w13, w2 = W13_cpu[e].double().numpy(), W2_cpu[e].double().numpy()
            t1 = time.perf_counter()
            y = O.expert_rows(x64[sorted_token[lo:hi]], w13, w2, "exact")
            if e < cfg.n_experts:
                y_routed[lo:hi] = y
            else:
                y_shared = y
            timed += time.perf_counter() - t1
        t2 = time.perf_counter()
        O.combine(y_routed, y_shared, pair_pos, r["gate"])
        O.bias_update(bias_cpu.numpy(), O.expert_counts(r["idx"], cfg.n_experts), cfg.T, cfg.top_k, cfg.gamma)
        timed += time.perf_counter() - t2
        del y_routed, y_shared
        steps += 1
    return {"value": round(cfg.T * steps / timed, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"fp64 oracle on {steps} whole {cfg.name} step(s) of fresh seeded batches: routing of "
                       f"{cfg.T} tokens, permutation, the SwiGLU FFN of all {cfg.n_experts + 1} experts on their "
                       f"{cfg.T * (cfg.top_k + 1)} rows, combine and bias update per step; {timed:.1f} s of oracle "
                       f"compute"),
            "seconds_measured": round(timed, 2)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1 "
                          "(the multi-GPU expert-parallel path is a design, not built)"}))
        sys.exit(2)
    import numpy as np
    import torch

    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload)
        return
    import sparse_moe_layer_sigmoid_amd as M
    from oracle import moe_oracle as O
    from sparse_moe_layer_sigmoid_amd import inputs as I

    M.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfgs = {c.name: c for c in I.CONFIGS.values()}
    main_e8m0 = args.workload.endswith("_e8m0")
    cfg = cfgs[args.workload[:-len("_e8m0")] if main_e8m0 else args.workload]
    t0 = time.time()
    log(f"[bench] generating V3 weights for {cfg.groups} experts ...")
    W13, W2 = I.gen_all_weights(cfg, dev)
    log(f"[bench] weights ready in {time.time() - t0:.1f}s")
    wr_cpu = I.gen_router(cfg).to(torch.bfloat16)
    wr = wr_cpu.to(dev)

    def measure(cfg, fp8, steps, warmup, n_batches=1, scales="f32"):
        bias_cpu = I.gen_bias(cfg)
        layer = M.MoELayer(wr, W13, W2, bias_cpu.to(dev), cfg.top_k, cfg.n_group, cfg.topk_group, fp8=fp8,
                           fp8_scales=scales)
        xs_cpu = [I.gen_x(cfg, step=None if n_batches == 1 else i) for i in range(n_batches)]
        xs = [x.to(dev) for x in xs_cpu]
        _, buf = layer.forward(xs[0], keep=True)
        counts0 = buf["expert_counts"].cpu().numpy()
        layer.bias.copy_(bias_cpu.to(dev))
        timer = KernelTimer(torch)
        ms = run_layer_steps(torch, M, layer, xs, steps, warmup, timer, cfg.gamma)
        return layer, xs_cpu, bias_cpu, counts0, ms, timer.mean_ms()

    # ---------------------------------------------------------------- headline workload
    fp8_main = cfg.dtype == "fp8"
    layer, xs_cpu, bias_cpu, counts0, ms, gu_ms = measure(cfg, fp8_main, args.steps, args.warmup,
                                                          scales="e8m0" if main_e8m0 else "f32")
    flops = O.layer_flops(cfg.T, cfg.d, cfg.n_experts, cfg.top_k, cfg.inter)
    tok_s = cfg.T / (ms / 1e3)
    gu_bytes = gate_up_bytes(cfg, counts0, fp8_main, 1 if main_e8m0 else 4)
    achieved = gu_bytes / (gu_ms / 1e3) / 1e9
    tag = f"gate_up_{args.workload}"
    line = {
        "metric": "MoE-layer tokens/s + % MFMA peak (T=4096 bf16, T=16384 fp8); decode GB/s",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8" if fp8_main else "bf16", "data": "synthetic (seeded N(0,1) x, random-init weights)",
        "config": {"workload": args.workload, "T": cfg.T, "d_model": cfg.d, "n_routed": cfg.n_experts, "n_shared": 1,
                   "top_k": cfg.top_k, "inter": cfg.inter, "n_group": cfg.n_group, "topk_group": cfg.topk_group,
                   "step": "route+permute+gateup_swiglu+down+combine+bias_update"},
        "tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "mfma_frac": round(flops / (ms / 1e3) / 1e12 / (FP8_PEAK_TFLOPS if fp8_main else BF16_PEAK_TFLOPS), 4),
        "roofline": {"kernel": "grouped_gemm gate/up + SwiGLU", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(tag), "avg_launch_ms": round(gu_ms, 4),
                     "algorithmic_bytes_per_launch": int(gu_bytes)},
    }
    log(f"[bench] {args.workload}: {ms:.3f} ms/step, {tok_s:,.0f} tok/s, gate/up {gu_ms:.3f} ms ({achieved:.0f} GB/s)")

    # ---------------------------------------------------------------- secondary workloads
    if not args.no_secondary:
        sec = []
        c3 = I.V3_FP8
        l3, _, _, counts3, ms3, gu3 = measure(c3, True, max(5, args.steps // 2), 3)
        f3 = O.layer_flops(c3.T, c3.d, c3.n_experts, c3.top_k, c3.inter)
        fl3 = 4 * c3.rows * c3.d * c3.inter
        sec.append({"workload": c3.name, "dtype": "fp8", "ms_per_step": round(ms3, 4),
                    "tokens_per_s": round(c3.T / (ms3 / 1e3), 1), "tflops": round(f3 / (ms3 / 1e3) / 1e12, 2),
                    "mfma_frac_fp8_peak": round(f3 / (ms3 / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                    "gate_up_ms": round(gu3, 4), "gate_up_traffic": measured_traffic(f"gate_up_{c3.name}"),
                    "gate_up_mfma_frac": round(fl3 / (gu3 / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4)})
        log(f"[bench] {c3.name}: {ms3:.3f} ms/step, gate/up {gu3:.3f} ms")
        # its backward on the FP8 path (E4M3 Dgrad and Wgrad)
        x3 = I.gen_x(c3).to(dev)
        _, buf3 = l3.forward(x3, keep=True)
        d3 = I.gen_normal(c3.seed + 900, (c3.T, c3.d), 1.0).to(dev)
        g3 = l3.backward(d3, buf3)  # warm-up; makes the transposed E4M3 weights once
        keep3 = {"dw13": g3["dw13"], "dw2": g3["dw2"]}
        del g3
        torch.cuda.synchronize()
        s3, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s3.record()
        for _ in range(3):
            g3 = l3.backward(d3, buf3, keep3)
            del g3
        e3.record()
        torch.cuda.synchronize()
        ms3b = s3.elapsed_time(e3) / 3
        fb3 = 2 * f3 + 4 * c3.rows * c3.d * c3.inter
        sec.append({"workload": c3.name + "_backward", "dtype": "fp8", "ms_per_step": round(ms3b, 4),
                    "tokens_per_s": round(c3.T / (ms3b / 1e3), 1), "tflops": round(fb3 / (ms3b / 1e3) / 1e12, 2),
                    "mfma_frac_fp8_peak": round(fb3 / (ms3b / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                    "note": "E4M3 Dgrad and Wgrad (1x128 / 128x128 scales, transposed operands quantised); f32 "
                            "weight gradients"})
        log(f"[bench] {c3.name}_backward: {ms3b:.3f} ms per backward")
        del l3, buf3, d3, keep3, x3
        torch.cuda.empty_cache()
        # the same layer with power-of-two (E8M0) tile scales applied by the matrix cores
        l3e, _, _, _, ms3e, gu3e = measure(c3, True, max(5, args.steps // 2), 3, scales="e8m0")
        sec.append({"workload": c3.name + "_e8m0", "dtype": "fp8", "scales": "e8m0", "ms_per_step": round(ms3e, 4),
                    "tokens_per_s": round(c3.T / (ms3e / 1e3), 1), "tflops": round(f3 / (ms3e / 1e3) / 1e12, 2),
                    "mfma_frac_fp8_peak": round(f3 / (ms3e / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                    "gate_up_ms": round(gu3e, 4),
                    "gate_up_traffic": measured_traffic(f"gate_up_{c3.name}_e8m0"),
                    "gate_up_mfma_frac": round(fl3 / (gu3e / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4)})
        log(f"[bench] {c3.name}_e8m0: {ms3e:.3f} ms/step, gate/up {gu3e:.3f} ms")
        del l3e
        # the backward pass of the headline layer (bf16): gradients of x, the router and every
        # expert's weights for a seeded d_out
        lb = M.MoELayer(wr, W13, W2, bias_cpu.to(dev), cfg.top_k, cfg.n_group, cfg.topk_group)
        xb = xs_cpu[0].to(dev)
        _, bufb = lb.forward(xb, keep=True)
        d_out = I.gen_normal(cfg.seed + 900, (cfg.T, cfg.d), 1.0).to(dev)
        gb = lb.backward(d_out, bufb)  # warm-up; makes the transposed weight copies once
        keep_g = {"dw13": gb["dw13"], "dw2": gb["dw2"]}  # weight gradients reused across steps
        del gb
        torch.cuda.synchronize()
        nb = 3
        sb, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sb.record()
        for _ in range(nb):
            gb = lb.backward(d_out, bufb, keep_g)
            del gb
        eb.record()
        torch.cuda.synchronize()
        msb = sb.elapsed_time(eb) / nb
        fb = 2 * O.layer_flops(cfg.T, cfg.d, cfg.n_experts, cfg.top_k, cfg.inter) + 4 * cfg.rows * cfg.d * cfg.inter
        sec.append({"workload": cfg.name + "_backward", "dtype": "bf16", "ms_per_step": round(msb, 4),
                    "tokens_per_s": round(cfg.T / (msb / 1e3), 1), "tflops": round(fb / (msb / 1e3) / 1e12, 2),
                    "mfma_frac_bf16_peak": round(fb / (msb / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                    "note": "dx, dW_r, dW13, dW2 (f32); gate/up products recomputed; weight-transpose copies made "
                            "once, outside the timed region"})
        log(f"[bench] {cfg.name}_backward: {msb:.3f} ms per backward")
        del lb, bufb, d_out, keep_g
        torch.cuda.empty_cache()
        c2 = I.V3_GROUP
        l2, _, _, _, ms2, _ = measure(c2, False, max(5, args.steps // 2), 3)
        f2 = O.layer_flops(c2.T, c2.d, c2.n_experts, c2.top_k, c2.inter)
        sec.append({"workload": c2.name, "dtype": "bf16", "ms_per_step": round(ms2, 4),
                    "tokens_per_s": round(c2.T / (ms2 / 1e3), 1), "tflops": round(f2 / (ms2 / 1e3) / 1e12, 2),
                    "mfma_frac_bf16_peak": round(f2 / (ms2 / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)})
        log(f"[bench] {c2.name}: {ms2:.3f} ms/step")
        del l2
        c4 = I.V3_DECODE
        n4 = args.decode_steps or c4.steps
        bias4 = I.gen_bias(c4)
        l4 = M.MoELayer(wr, W13, W2, bias4.to(dev), c4.top_k, fp8=True)
        xs4 = [I.gen_x(c4, step=i).to(dev) for i in range(n4)]
        for i in range(3):
            l4.forward(xs4[i])
        l4.bias.copy_(bias4.to(dev))
        torch.cuda.synchronize()
        # the steps run back to back as in a decode loop (no host synchronisation between them):
        # each is bracketed by its own events and its expert loads are copied into a device-side
        # history, read once the loop has finished
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n4)]
        hist = torch.empty((n4, c4.n_experts), dtype=torch.int32, device=dev)
        for i in range(n4):
            ev[i][0].record()
            _, buf = l4.forward(xs4[i], update_bias=True, gamma=c4.gamma, keep=True)
            ev[i][1].record()
            hist[i].copy_(buf["expert_counts"])
        torch.cuda.synchronize()
        loads, gbs, times = [], [], []
        for i, cnt in enumerate(hist.cpu().numpy()):
            t = ev[i][0].elapsed_time(ev[i][1])
            loads.append(float(cnt.max() / cnt.mean()))
            gbs.append(step_bytes(c4, cnt, True) / (t / 1e3) / 1e9)
            times.append(t)
        sec.append({"workload": c4.name, "dtype": "fp8", "steps": n4,
                    "ms_per_step_median": round(float(np.median(times)), 4),
                    "gbs_median": round(float(np.median(gbs)), 1),
                    "hbm_frac_median": round(float(np.median(gbs)) / HBM_PEAK_GBS, 4),
                    "gbs_median_first10": round(float(np.median(gbs[:10])), 1),
                    "gbs_median_last10": round(float(np.median(gbs[-10:])), 1),
                    "max_over_mean_load_first": round(loads[0], 3), "max_over_mean_load_last": round(loads[-1], 3),
                    "max_over_mean_load_series_every10": [round(v, 3) for v in loads[::10]]})
        log(f"[bench] {c4.name}: median {np.median(times):.3f} ms, {np.median(gbs):.0f} GB/s, load {loads[0]:.2f}->{loads[-1]:.2f}")
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(cfg, wr_cpu, bias_cpu, W13.cpu(), W2.cpu())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
