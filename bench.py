"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-secondary]
                    [--no-cpu-baseline]
    python bench.py --ceilings     (the chip's measured ceilings; no layer)
    python bench.py --backward-only   (the two backward workloads alone)
    python bench.py --t-sweep         (the layer at T = 256 .. 32768, bf16 and E4M3)

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
    p.add_argument("--decode-sweep-steps", type=int, default=20)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first copy 1 GiB device-to-device twice (the reference dispatch for HBM counters)")
    p.add_argument("--backward-only", action="store_true",
                   help="time only the two backward workloads (bf16 T = 4096, E4M3 T = 16384) and print one JSON line")
    p.add_argument("--t-sweep", action="store_true",
                   help="time the V3-shaped layer (bf16 and E4M3, bias update on) at T = 256 .. 32768 and print "
                        "one JSON line")
    p.add_argument("--ceilings", action="store_true",
                   help="run the ceiling micro-benchmarks (HBM read, DMA read in the GEMM's pattern, copy, "
                        "LDS read, matrix cores, fp32 FMA) instead of the layer and print one JSON line")
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


def run_layer_steps(torch, M, layer, xs, steps, warmup, timers, gamma, update_bias=True):
    """Warm up, then time `steps` forwards (events on the current stream).  timers: dict of
    KernelTimer for "gate_up", "down" and "combine", filled during the timed steps."""
    import sparse_moe_layer_sigmoid_amd.layer as layer_mod
    L = layer_mod.L
    orig_gg, orig_cb = L.moe_grouped_gemm, L.moe_combine
    state = {"timing": False}

    def gg(*a, **kw):
        if state["timing"]:
            return timers["gate_up" if kw.get("swiglu") else "down"].wrap(orig_gg, *a, **kw)
        return orig_gg(*a, **kw)

    def cb(*a, **kw):
        if state["timing"]:
            return timers["combine"].wrap(orig_cb, *a, **kw)
        return orig_cb(*a, **kw)

    L.moe_grouped_gemm, L.moe_combine = gg, cb
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
        L.moe_grouped_gemm, L.moe_combine = orig_gg, orig_cb


def kernel_fractions(cfg, counts, fp8, e8m0, km):
    """Per-kernel achieved rates against their roofline: the GEMMs against the matrix-core
    peak of their dtype (and HBM), the combine against HBM."""
    fl_gu = 4 * cfg.rows * cfg.d * cfg.inter
    fl_dn = 2 * cfg.rows * cfg.d * cfg.inter
    peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    out = {}
    for name, fl, by in (("gate_up", fl_gu, gate_up_bytes(cfg, counts, fp8, 1 if e8m0 else 4)),
                         ("down", fl_dn, down_bytes(cfg, counts, fp8))):
        ms = km[name]
        tf = fl / (ms / 1e3) / 1e12
        gbs = by / (ms / 1e3) / 1e9
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "mfma_frac": round(tf / peak, 4),
                     "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    ms = km["combine"]
    gbs = combine_bytes(cfg) / (ms / 1e3) / 1e9
    out["combine"] = {"ms": round(ms, 4), "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def gate_up_bytes(cfg, counts_np, fp8: bool, scale_bytes: int = 4):
    """Algorithmic HBM bytes of one gate/up launch: the W13 of every expert with at least one
    row (plus the shared one) read once, the input x read once (T rows: the gather of a
    token's K + 1 rows re-reads it from cache, not from HBM), h written once (fp8: with
    their scales, scale_bytes each)."""
    esz = 1 if fp8 else 2
    sb = scale_bytes if fp8 else 0
    active = int((counts_np > 0).sum()) + 1
    w = active * 2 * cfg.inter * cfg.d * esz + active * (2 * cfg.inter // 128) * (cfg.d // 128) * sb
    a = cfg.T * cfg.d * esz + cfg.T * (cfg.d // 128) * sb
    h = cfg.rows * cfg.inter * esz + cfg.rows * (cfg.inter // 128) * sb
    return w + a + h


def down_bytes(cfg, counts_np, fp8: bool):
    """Algorithmic HBM bytes of one down launch: the W2 of every active expert (and the
    shared one) read once, h read once, routed y written in bf16 and the shared y in f32."""
    esz = 1 if fp8 else 2
    sb = 4 if fp8 else 0
    active = int((counts_np > 0).sum()) + 1
    w = active * cfg.d * cfg.inter * esz + active * (cfg.d // 128) * (cfg.inter // 128) * sb
    h = cfg.rows * cfg.inter * esz + cfg.rows * (cfg.inter // 128) * sb
    return w + h + cfg.T * cfg.top_k * cfg.d * 2 + cfg.T * cfg.d * 4


def combine_bytes(cfg):
    """Algorithmic HBM bytes of one combine: the K routed rows (bf16) and the shared row (f32)
    of every token read once, the bf16 output written once."""
    return cfg.T * cfg.top_k * cfg.d * 2 + cfg.T * cfg.d * 4 + cfg.T * cfg.d * 2


def step_bytes(cfg, counts_np, fp8: bool):
    """Algorithmic bytes of one whole-layer step (weights of active experts + router once,
    x in, out written): the decode-shaped run's GB/s numerator."""
    esz = 1 if fp8 else 2
    active = int((counts_np > 0).sum()) + 1
    w = active * 3 * cfg.inter * cfg.d * esz
    if fp8:
        w += active * ((2 * cfg.inter // 128) * (cfg.d // 128) + (cfg.d // 128) * (cfg.inter // 128)) * 4
    return w + cfg.n_experts * cfg.d * 2 + 2 * cfg.T * cfg.d * 2


def gate_up_roofline(flop, nbytes, ms, fp8: bool):
    """Roofline object of the gate/up launch: against the matrix-core peak of its dtype when its
    arithmetic intensity (algorithmic flop per algorithmic byte) lies above that peak's ridge
    point (peak flop/s over the 8 TB/s HBM peak: 312 flop/B for bf16, 625 for E4M3), else
    against the HBM peak."""
    peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    name = "grouped_gemm gate/up + SwiGLU" + (" (E4M3)" if fp8 else "")
    common = {"traffic": None, "avg_launch_ms": round(ms, 4), "algorithmic_flop_per_launch": int(flop),
              "algorithmic_bytes_per_launch": int(nbytes)}
    if flop / nbytes > ridge:
        achieved = flop / (ms / 1e3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), **common}
    achieved = nbytes / (ms / 1e3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), **common}


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
    # template arguments <..., input kind (0 bf16, 1 E4M3 + f32 scales, 2 E4M3 + E8M0), SwiGLU, output,
    # pre-activation output (the inference forward: false)>
    kind = 2 if workload.endswith("_e8m0") else (1 if "fp8" in workload else 0)
    want = f"{kind}, true, {2 if kind else 0}, false>"
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
            "seconds_measured": round(timed, 2), "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name (first processor entry), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def decode_skew_sweep(torch, M, I, wr, W13, W2, dev, steps):
    """The decode shape (T = 256, E4M3 path) under three fixed routing skews, no bias update:
    a zero bias (the router's own spread), the Zipf(1.1) popularity bias, and +10 on experts
    0..7 (every token picks the same 8 experts: the hottest load the method allows).  Each
    step is timed alone (events around it, steps back to back); reported per skew: median
    time, tokens/s, the algorithmic bytes of the experts that receive tokens over the time,
    max/mean load and the active-expert count."""
    import numpy as np
    c4 = I.V3_DECODE
    xs = [I.gen_x(c4, step=i).to(dev) for i in range(steps)]
    zipf = I.gen_bias(c4)
    hot = torch.zeros(c4.n_experts, dtype=torch.float32)
    hot[:c4.top_k] = 10.0
    out = {"workload": c4.name + "_skew_sweep", "dtype": "fp8", "steps": steps}
    layer = M.MoELayer(wr, W13, W2, zipf.to(dev), c4.top_k, fp8=True)
    for name, b in (("zero_bias", torch.zeros(c4.n_experts)), ("zipf_1.1", zipf), ("hot8_plus10", hot)):
        layer.bias = b.to(dev).clone()
        for i in range(3):
            layer.forward(xs[i])
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        hist = torch.empty((steps, c4.n_experts), dtype=torch.int32, device=dev)
        for i in range(steps):
            ev[i][0].record()
            _, buf = layer.forward(xs[i], keep=True)
            ev[i][1].record()
            hist[i].copy_(buf["expert_counts"])
        torch.cuda.synchronize()
        h = hist.cpu().numpy()
        t = np.array([a.elapsed_time(b_) for a, b_ in ev])
        by = np.array([step_bytes(c4, c, True) for c in h])
        out[name] = {"ms_median": round(float(np.median(t)), 4),
                     "tokens_per_s": round(c4.T / (float(np.median(t)) / 1e3), 1),
                     "gbs_median": round(float(np.median(by / (t / 1e3) / 1e9)), 1),
                     "bytes_per_step_median": int(np.median(by)),
                     "max_over_mean_load": round(float(np.median(h.max(axis=1) / h.mean(axis=1))), 2),
                     "active_experts_median": int(np.median((h > 0).sum(axis=1)))}
        log(f"[bench] decode skew {name}: {out[name]}")
    return out


def time_backward(torch, layer, x, d_out, n=3):
    """Mean times of n backward passes of `layer` for the forward of x (kept), after one warm-up
    pass that also makes the transposed weight copies (the weight gradients are reused), and of
    n training forwards (train=True: the forward that also stores what the backward takes, the
    gate/up products a | c among it)."""
    _, buf = layer.forward(x, train=True)
    g = layer.backward(d_out, buf)
    keep = {"dw13": g["dw13"], "dw2": g["dw2"]}
    del g
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        g = layer.backward(d_out, buf, keep)
        del g
    e.record()
    torch.cuda.synchronize()
    ms_bwd = s.elapsed_time(e) / n
    del buf
    s.record()
    for _ in range(n):
        _, buf = layer.forward(x, train=True)
        del buf
    e.record()
    torch.cuda.synchronize()
    return ms_bwd, s.elapsed_time(e) / n


def backward_record(name, dtype, T, times, flops, peak, note):
    ms, ms_fwd = times
    return {"workload": name + "_backward", "dtype": dtype, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(T / (ms / 1e3), 1), "tflops": round(flops / (ms / 1e3) / 1e12, 2),
            f"mfma_frac_{dtype}_peak": round(flops / (ms / 1e3) / 1e12 / peak, 4),
            "training_forward_ms": round(ms_fwd, 4), "note": note}


BWD_NOTE_FP8 = ("E4M3 Dgrad and Wgrad (1x128 / 128x128 scales, transposed operands quantised); f32 weight gradients; "
                "gate/up products a | c stored by the training forward (training_forward_ms), not recomputed")
BWD_NOTE_BF16 = ("dx, dW_r, dW13, dW2 (f32); gate/up products a | c stored by the training forward "
                 "(training_forward_ms), not recomputed; weight-transpose copies made once, outside the timed region")


def layer_flops(c):
    """Algorithmic flops of one forward: the router (2 T d N) plus a SwiGLU expert (6 d I) per
    token for each of its top_k routed experts and the shared one."""
    return 2 * c.T * c.d * c.n_experts + 6 * c.d * c.inter * c.T * (c.top_k + 1)


def backward_flops(c):
    """Algorithmic flops of one backward: twice the forward's (Dgrad and Wgrad)."""
    return 2 * layer_flops(c)


def run_backward_only(torch, M, I, dev):
    """The two backward workloads alone (bf16 at T = 4096, E4M3 at T = 16384)."""
    out = []
    for c, fp8 in ((I.V3_BF16, False), (I.V3_FP8, True)):
        log(f"[bench] {c.name}_backward: weights ...")
        W13, W2 = I.gen_all_weights(c, dev)
        wr = I.gen_router(c).to(torch.bfloat16).to(dev)
        layer = M.MoELayer(wr, W13, W2, I.gen_bias(c).to(dev), c.top_k, c.n_group, c.topk_group, fp8=fp8)
        x = I.gen_x(c).to(dev)
        d_out = I.gen_normal(c.seed + 900, (c.T, c.d), 1.0).to(dev)
        ms = time_backward(torch, layer, x, d_out)
        out.append(backward_record(c.name, "fp8" if fp8 else "bf16", c.T, ms, backward_flops(c),
                                   FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS,
                                   BWD_NOTE_FP8 if fp8 else BWD_NOTE_BF16))
        log(f"[bench] {c.name}_backward: {ms[0]:.3f} ms per backward, {ms[1]:.3f} ms per training forward")
        del layer, W13, W2, x, d_out
        torch.cuda.empty_cache()
    return out


def run_t_sweep(torch, M, I, dev, steps=10, warmup=3):
    """The V3-shaped layer against the batch size: for each T the same seeded x every step,
    `warmup` untimed and `steps` timed forwards with the bias update (events on the stream),
    the bias restored between sizes."""
    c = I.V3_BF16
    W13, W2 = I.gen_all_weights(c, dev)
    wr = I.gen_router(c).to(torch.bfloat16).to(dev)
    out = []
    for fp8 in (False, True):
        layer = M.MoELayer(wr, W13, W2, I.gen_bias(c).to(dev), c.top_k, fp8=fp8)
        b0 = layer.bias.clone()
        for T in (256, 1024, 2048, 4096, 8192, 16384, 32768):
            cfg = I.small(c, T=T, name=f"v3_T{T}")
            x = I.gen_x(cfg).to(dev)
            for _ in range(warmup):
                layer.forward(x, update_bias=True, gamma=c.gamma)
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(steps):
                layer.forward(x, update_bias=True, gamma=c.gamma)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e) / steps
            layer.bias.copy_(b0)
            fl = layer_flops(cfg)
            peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
            out.append({"dtype": "fp8" if fp8 else "bf16", "T": T, "ms_per_step": round(ms, 4),
                        "tokens_per_s": round(T / (ms / 1e3), 1), "tflops": round(fl / (ms / 1e3) / 1e12, 1),
                        "mfma_frac": round(fl / (ms / 1e3) / 1e12 / peak, 4)})
            log(f"[bench] t-sweep {out[-1]}")
            del x
            torch.cuda.empty_cache()
        del layer
        torch.cuda.empty_cache()
    return out


def run_ceilings(torch, dev):
    """The chip's measured ceilings from libmoe_ceilings.so: each probe warmed up twice, then
    timed five times with HIP events on the stream it runs on (the best run is reported);
    per-clock figures from the probes' own s_memtime cycle counts (median over workgroups)."""
    path = os.path.join(ROOT, "sparse_moe_layer_sigmoid_amd", "libmoe_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: python -m sparse_moe_layer_sigmoid_amd.build")
    lib = ctypes.CDLL(path)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
    lib.moe_ceil_hbm_read.argtypes = [P, S, P, S, I32, P]
    lib.moe_ceil_dma_read.argtypes = [P, I64, I32, P, S, I32, P]
    lib.moe_ceil_dma_resident.argtypes = [I32, P, I32, I32, I32, P, P, S, I32, P]
    lib.moe_ceil_dma_read_ring.argtypes = [I32, P, I64, I32, P, S, I32, P]
    lib.moe_ceil_lds_read.argtypes = [I32, I32, P, P, S, I32, P]
    lib.moe_ceil_mfma.argtypes = [I32, I32, P, P, S, I32, P]
    lib.moe_ceil_valu.argtypes = [I32, P, P, S, I32, P]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    sink = torch.empty(cus * 16 * 512, dtype=torch.int32, device=dev)
    cycles = torch.empty(cus, dtype=torch.int64, device=dev)
    sk, skn, cy = sink.data_ptr(), sink.numel(), cycles.data_ptr()

    def timed(call, reps=5, warm=2):
        for _ in range(warm):
            rc = call()
            if rc != 0:
                raise RuntimeError(f"ceiling probe returned {rc}")
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        return best

    def med_cycles():
        return float(cycles.cpu().double().median())

    out = {"cus": cus}
    buf = torch.empty(8 << 30, dtype=torch.uint8, device=dev)
    rd = {}
    for mult in (4, 8, 16):
        ms = timed(lambda: lib.moe_ceil_hbm_read(buf.data_ptr(), buf.numel(), sk, skn, cus * mult, sp))
        rd[f"grid_{mult}x"] = round(buf.numel() / (ms / 1e3) / 1e9, 1)
    out["hbm_read_vector_GBs"] = {"bytes": buf.numel(), **rd, "best": max(rd.values())}
    row_bytes = 7168 * 2
    rows = buf.numel() // row_bytes // 256 * 256
    ms = timed(lambda: lib.moe_ceil_dma_read(buf.data_ptr(), rows, row_bytes, sk, skn, cus, sp))
    out["hbm_read_dma_gemm_pattern_GBs"] = {"rows": rows, "row_bytes": row_bytes, "grid": cus,
                                            "GBs": round(rows * row_bytes / (ms / 1e3) / 1e9, 1)}
    ring = {}
    for slots in (2, 3, 4, 5):  # slots - 1 steps of 32 KB in flight per CU
        ms = timed(lambda: lib.moe_ceil_dma_read_ring(slots, buf.data_ptr(), rows, row_bytes, sk, skn, cus, sp))
        ring[f"slots_{slots}"] = round(rows * row_bytes / (ms / 1e3) / 1e9, 1)
    out["hbm_read_dma_by_ring_depth_GBs"] = ring
    # the same step pattern over working sets held by one cache level: 8 row blocks of 256 rows x
    # 2 KB read by every CU (4 MB: in each XCD's L2), and one 256-row x 1 KB block per CU (8 MB
    # per XCD, past its 4 MB L2; 64 MB in all, inside the Infinity Cache), by direct-to-LDS DMA
    # and by vector loads into registers
    res = {}
    for label, n_blocks, rbytes, steps in (("l2", 8, 2048, 1800), ("infinity_cache", cus, 1024, 240)):
        for mode, how in ((0, "dma"), (1, "vector_loads")):
            ms = timed(lambda: lib.moe_ceil_dma_resident(mode, buf.data_ptr(), n_blocks, rbytes, steps, cy, sk, skn,
                                                         cus, sp))
            per_cu = steps * 256 * 128
            res[f"{label}_{how}"] = {"B_per_clk_per_CU": round(per_cu / med_cycles(), 1),
                                     "TBs_chip": round(per_cu * cus / (ms / 1e3) / 1e12, 2)}
    out["resident_read_gemm_pattern"] = res
    half = buf.numel() // 2
    src, dst = buf[:half], buf[half:]
    ms = timed(lambda: (dst.copy_(src), 0)[1])
    out["d2d_copy_GBs"] = {"bytes_each_way": half, "GBs_read_plus_write": round(2 * half / (ms / 1e3) / 1e9, 1)}
    del buf, src, dst
    clocks = []
    for width in (16, 8):
        iters = 16384
        ms = timed(lambda: lib.moe_ceil_lds_read(width, iters, cy, sk, skn, cus, sp))
        per_block = 512 * width * iters
        c = med_cycles()
        clocks.append(c / (ms * 1e6))
        out[f"lds_read_b{width * 8}"] = {"B_per_clk_per_CU": round(per_block / c, 1),
                                          "TBs_chip": round(per_block * cus / (ms / 1e3) / 1e12, 2)}
    for kind, name, fl in ((0, "mfma_bf16_16x16x32", 2 * 16 * 16 * 32), (1, "mfma_e4m3_16x16x128", 2 * 16 * 16 * 128),
                           (2, "mfma_e4m3_16x16x128_promoted", 2 * 16 * 16 * 128)):
        iters = 2048
        ms = timed(lambda: lib.moe_ceil_mfma(kind, iters, cy, sk, skn, cus, sp))
        flops = cus * 8 * iters * 8 * fl
        c = med_cycles()
        clocks.append(c / (ms * 1e6))
        out[name] = {"TFLOPs": round(flops / (ms / 1e3) / 1e12, 1),
                     "flop_per_clk_per_CU": round(flops / cus / c, 1)}
    iters = 65536
    ms = timed(lambda: lib.moe_ceil_valu(iters, cy, sk, skn, cus, sp))
    flops = cus * 512 * iters * 8 * 2
    c = med_cycles()
    clocks.append(c / (ms * 1e6))
    out["valu_fp32_fma"] = {"TFLOPs": round(flops / (ms / 1e3) / 1e12, 1), "flop_per_clk_per_CU": round(flops / cus / c, 1)}
    out["shader_clock_GHz_per_probe"] = [round(x, 3) for x in clocks]
    # the vendor library's dense GEMMs at the gate/up shape of 16384 tokens x 8 + 1 experts
    # (one M x 2I x d product), for comparison with the grouped kernels: bf16 through
    # torch.matmul, E4M3 with one scale per tensor through torch._scaled_mm
    Mr, Nr, Kr = 147456, 4096, 7168
    lib_gemm = {"M": Mr, "N": Nr, "K": Kr}
    a = torch.randn(Mr, Kr, device=dev, dtype=torch.bfloat16)
    b = torch.randn(Nr, Kr, device=dev, dtype=torch.bfloat16)
    ms = timed(lambda: (torch.matmul(a, b.t()), 0)[1], reps=3, warm=1)
    lib_gemm["bf16_TFLOPs"] = round(2 * Mr * Nr * Kr / (ms / 1e3) / 1e12, 1)
    try:
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
        one = torch.ones((), device=dev, dtype=torch.float32)
        ms = timed(lambda: (torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 0)[1],
                   reps=3, warm=1)
        lib_gemm["e4m3_tensor_scaled_TFLOPs"] = round(2 * Mr * Nr * Kr / (ms / 1e3) / 1e12, 1)
    except Exception as e:  # the library may not offer this product on the installed stack
        lib_gemm["e4m3_tensor_scaled_TFLOPs"] = None
        lib_gemm["e4m3_error"] = str(e)[:200]
    out["library_dense_gemm"] = lib_gemm
    return out


def measured_peaks(torch, dev):
    """A short subset of the ceiling probes, for the bench line's secondary denominators: the
    HBM read rate of direct-to-LDS DMA in the grouped GEMM's weight pattern (8 GiB) and the
    bf16 / E4M3 matrix-core rates from registers."""
    path = os.path.join(ROOT, "sparse_moe_layer_sigmoid_amd", "libmoe_ceilings.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
    lib.moe_ceil_dma_read.argtypes = [P, I64, I32, P, S, I32, P]
    lib.moe_ceil_mfma.argtypes = [I32, I32, P, P, S, I32, P]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sp = torch.cuda.current_stream().cuda_stream
    sink = torch.empty(cus * 512, dtype=torch.int32, device=dev)
    cycles = torch.empty(cus, dtype=torch.int64, device=dev)

    def best_ms(call, reps=5):
        call()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = call()
            b.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"ceiling probe returned {rc}")
            best = a.elapsed_time(b) if best is None else min(best, a.elapsed_time(b))
        return best

    row_bytes = 7168 * 2
    rows = (8 << 30) // row_bytes // 256 * 256
    buf = torch.empty(rows * row_bytes, dtype=torch.uint8, device=dev)
    ms = best_ms(lambda: lib.moe_ceil_dma_read(buf.data_ptr(), rows, row_bytes, sink.data_ptr(), sink.numel(), cus, sp))
    out = {"hbm_read_dma_GBs": round(rows * row_bytes / (ms / 1e3) / 1e9, 1)}
    del buf
    for kind, name, fl in ((0, "mfma_bf16_TFLOPs", 2 * 16 * 16 * 32), (1, "mfma_e4m3_TFLOPs", 2 * 16 * 16 * 128)):
        iters = 2048
        ms = best_ms(lambda: lib.moe_ceil_mfma(kind, iters, cycles.data_ptr(), sink.data_ptr(), sink.numel(), cus, sp))
        out[name] = round(cus * 8 * iters * 8 * fl / (ms / 1e3) / 1e12, 1)
    out["source"] = "bench.py measured_peaks (probes of sparse_moe_layer_sigmoid_amd/ceilings/ceilings.hip)"
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this implementation runs on one GPU only: --gpus must be 1 "
                          "(the multi-GPU expert-parallel path is a design, not built)"}))
        sys.exit(2)
    import numpy as np
    import torch

    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload)
        return
    import sparse_moe_layer_sigmoid_amd as M
    from sparse_moe_layer_sigmoid_amd import inputs as I

    M.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.ceilings:
        print(json.dumps({"ceilings": run_ceilings(torch, dev), "device": torch.cuda.get_device_name(dev)}),
              flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": run_backward_only(torch, M, I, dev)}), flush=True)
        return
    if args.t_sweep:
        print(json.dumps({"t_sweep": run_t_sweep(torch, M, I, dev)}), flush=True)
        return
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
        timers = {k: KernelTimer(torch) for k in ("gate_up", "down", "combine")}
        ms = run_layer_steps(torch, M, layer, xs, steps, warmup, timers, cfg.gamma)
        km = {k: t.mean_ms() for k, t in timers.items()}
        kf = kernel_fractions(cfg, counts0, fp8, scales == "e8m0", km)
        return layer, xs_cpu, bias_cpu, counts0, ms, km["gate_up"], kf

    # ---------------------------------------------------------------- headline workload
    fp8_main = cfg.dtype == "fp8"
    layer, xs_cpu, bias_cpu, counts0, ms, gu_ms, kf = measure(cfg, fp8_main, args.steps, args.warmup,
                                                              scales="e8m0" if main_e8m0 else "f32")
    flops = layer_flops(cfg)
    tok_s = cfg.T / (ms / 1e3)
    gu_bytes = gate_up_bytes(cfg, counts0, fp8_main, 1 if main_e8m0 else 4)
    gu_flop = 4 * cfg.rows * cfg.d * cfg.inter
    tag = f"gate_up_{args.workload}"
    roofline = gate_up_roofline(gu_flop, gu_bytes, gu_ms, fp8_main)
    roofline["traffic"] = measured_traffic(tag)
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
        "roofline": roofline,
        "kernels": kf,
    }
    log(f"[bench] {args.workload}: {ms:.3f} ms/step, {tok_s:,.0f} tok/s, gate/up {gu_ms:.3f} ms ({roofline['achieved']:.0f} "
        f"{roofline['unit']}), down {kf['down']['ms']:.3f} ms, combine {kf['combine']['ms']:.3f} ms")

    # ---------------------------------------------------------------- secondary workloads
    if not args.no_secondary:
        sec = []
        c3 = I.V3_FP8
        l3, _, _, counts3, ms3, gu3, kf3 = measure(c3, True, max(5, args.steps // 2), 3)
        f3 = layer_flops(c3)
        fl3 = 4 * c3.rows * c3.d * c3.inter
        sec.append({"workload": c3.name, "dtype": "fp8", "ms_per_step": round(ms3, 4),
                    "tokens_per_s": round(c3.T / (ms3 / 1e3), 1), "tflops": round(f3 / (ms3 / 1e3) / 1e12, 2),
                    "mfma_frac_fp8_peak": round(f3 / (ms3 / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                    "gate_up_ms": round(gu3, 4), "gate_up_traffic": measured_traffic(f"gate_up_{c3.name}"),
                    "gate_up_mfma_frac": round(fl3 / (gu3 / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4), "kernels": kf3})
        log(f"[bench] {c3.name}: {ms3:.3f} ms/step, gate/up {gu3:.3f} ms")
        # its backward on the FP8 path (E4M3 Dgrad and Wgrad)
        x3 = I.gen_x(c3).to(dev)
        d3 = I.gen_normal(c3.seed + 900, (c3.T, c3.d), 1.0).to(dev)
        ms3b = time_backward(torch, l3, x3, d3)
        sec.append(backward_record(c3.name, "fp8", c3.T, ms3b, backward_flops(c3), FP8_PEAK_TFLOPS, BWD_NOTE_FP8))
        log(f"[bench] {c3.name}_backward: {ms3b[0]:.3f} ms per backward, {ms3b[1]:.3f} ms per training forward")
        del l3, d3, x3
        torch.cuda.empty_cache()
        # the same layer with power-of-two (E8M0) tile scales applied by the matrix cores
        l3e, _, _, _, ms3e, gu3e, kf3e = measure(c3, True, max(5, args.steps // 2), 3, scales="e8m0")
        sec.append({"workload": c3.name + "_e8m0", "dtype": "fp8", "scales": "e8m0", "ms_per_step": round(ms3e, 4),
                    "tokens_per_s": round(c3.T / (ms3e / 1e3), 1), "tflops": round(f3 / (ms3e / 1e3) / 1e12, 2),
                    "mfma_frac_fp8_peak": round(f3 / (ms3e / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                    "gate_up_ms": round(gu3e, 4),
                    "gate_up_traffic": measured_traffic(f"gate_up_{c3.name}_e8m0"),
                    "gate_up_mfma_frac": round(fl3 / (gu3e / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4), "kernels": kf3e})
        log(f"[bench] {c3.name}_e8m0: {ms3e:.3f} ms/step, gate/up {gu3e:.3f} ms")
        del l3e
        # the backward pass of the headline layer (bf16): gradients of x, the router and every
        # expert's weights for a seeded d_out
        lb = M.MoELayer(wr, W13, W2, bias_cpu.to(dev), cfg.top_k, cfg.n_group, cfg.topk_group)
        xb = xs_cpu[0].to(dev)
        d_out = I.gen_normal(cfg.seed + 900, (cfg.T, cfg.d), 1.0).to(dev)
        msb = time_backward(torch, lb, xb, d_out)
        sec.append(backward_record(cfg.name, "bf16", cfg.T, msb, backward_flops(cfg), BF16_PEAK_TFLOPS,
                                   BWD_NOTE_BF16))
        log(f"[bench] {cfg.name}_backward: {msb[0]:.3f} ms per backward, {msb[1]:.3f} ms per training forward")
        del lb, xb, d_out
        torch.cuda.empty_cache()
        c2 = I.V3_GROUP
        l2, _, _, _, ms2, _, kf2 = measure(c2, False, max(5, args.steps // 2), 3)
        f2 = layer_flops(c2)
        sec.append({"workload": c2.name, "dtype": "bf16", "ms_per_step": round(ms2, 4),
                    "tokens_per_s": round(c2.T / (ms2 / 1e3), 1), "tflops": round(f2 / (ms2 / 1e3) / 1e12, 2),
                    "mfma_frac_bf16_peak": round(f2 / (ms2 / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4), "kernels": kf2})
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
        loads, gbs, times, active = [], [], [], []
        for i, cnt in enumerate(hist.cpu().numpy()):
            t = ev[i][0].elapsed_time(ev[i][1])
            loads.append(float(cnt.max() / cnt.mean()))
            gbs.append(step_bytes(c4, cnt, True) / (t / 1e3) / 1e9)
            times.append(t)
            active.append(int((cnt > 0).sum()))
        sec.append({"workload": c4.name, "dtype": "fp8", "steps": n4,
                    "ms_per_step_median": round(float(np.median(times)), 4),
                    "gbs_median": round(float(np.median(gbs)), 1),
                    "hbm_frac_median": round(float(np.median(gbs)) / HBM_PEAK_GBS, 4),
                    "gbs_median_first10": round(float(np.median(gbs[:10])), 1),
                    "gbs_median_last10": round(float(np.median(gbs[-10:])), 1),
                    "max_over_mean_load_first": round(loads[0], 3), "max_over_mean_load_last": round(loads[-1], 3),
                    "per_step": {"max_over_mean_load": [round(v, 2) for v in loads],
                                 "active_experts": active, "gbs": [round(v) for v in gbs],
                                 "ms": [round(v, 3) for v in times]}})
        log(f"[bench] {c4.name}: median {np.median(times):.3f} ms, {np.median(gbs):.0f} GB/s, load {loads[0]:.2f}->{loads[-1]:.2f}")
        del l4, xs4, hist
        sec.append(decode_skew_sweep(torch, M, I, wr, W13, W2, dev, args.decode_sweep_steps))
        line["secondary"] = sec
        # the chip's measured ceilings as a second denominator for the roofline
        peaks = measured_peaks(torch, dev)
        if peaks:
            line["measured_peaks"] = peaks
            if roofline["bound"] == "mfma":
                ref = peaks["mfma_e4m3_TFLOPs"] if fp8_main else peaks["mfma_bf16_TFLOPs"]
            else:
                ref = peaks["hbm_read_dma_GBs"]
            line["roofline"]["frac_of_measured_peak"] = round(roofline["achieved"] / ref, 4)

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(cfg, wr_cpu, bias_cpu, W13.cpu(), W2.cpu())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
