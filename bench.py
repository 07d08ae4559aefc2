"""Benchmark of the routed int4 MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill512|prefill4096|stack1|stack16]

A step is one pass of the whole layer (route -> experts -> combine) over one
batch of synthetic input already resident in HBM:
  decode       T=1 token through one layer (Qwen3.6-35B-A3B shape: H=2048,
               E=256, top-8 + shared, I=512, int4 g64 experts, 8-bit router);
               steps rotate over --copies independent weight sets (3.6 GB by
               default) and 64 tokens so weights come from HBM, not cache;
  prefill512   T=512 tokens through one layer;
  prefill4096  T=4096 tokens, Zipf(1.1) logit bias (skewed expert loads);
  stack1/16    one decode step of T=1 / T=16 tokens through 40 stacked layers
               (one moe_decode_block launch per layer: RMSNorm, layer, residual).
The timed region replays HIP graphs of the step sequence (captured once): one
graph of min(K, 64) steps replayed K // that times, and one of the remaining steps.
The process prints one JSON line. Its headline is the chosen workload (decode by
default); "workloads" holds a record of the same form for each other workload
(skipped with --only), timed with the same step counts capped by that
workload's default. `roofline` covers the dominant stage: decode_layer_kernel for
T <= 16, the experts stage (moe_experts_prefill) for prefill, timed with HIP events
on the launch stream. `cpu_baseline` times the FP64 oracle on a bounded sample
(`cores`: BLAS threads it ran with; `host_cores`: the host's core count).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

EXPERT_BYTES = 1_769_472  # gate+up+down q and scale/bias for H=2048, I=512
# 8-bit experts: one code per byte and one (scale, bias) pair per 64 codes (the
# packed form carries one more word per group: 3,538,944 B)
EXPERT_BYTES_8BIT = 3 * 2048 * 512 + 3 * 2048 * 512 // 64 * 4
FP8_EXPERT_BYTES = 3 * 2048 * 512 + 4 * (2 * 512 + 2048)  # E4M3 codes and float row scales
FP8_PEAK_TFLOPS = 5000.0
ROUTER_BYTES = 559_232


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill512", "prefill4096", "stack1", "stack16", "decode_8bit",
                             "prefill512_8bit", "prefill512_fp8", "prefill4096_fp8"])
    ap.add_argument("--copies", type=int, default=8, help="independent weight sets for the decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="measure the chosen workload alone (no sub-records)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (counter calibration) and exit")
    ap.add_argument("--traffic-from", default=None, metavar="FETCH,WRITE,CAL_FETCH,CAL_WRITE",
                    help="rocprofv3 --pmc output folders of FETCH_SIZE and WRITE_SIZE runs of this workload and "
                         "of --copy-calibration; writes the scaled per-launch traffic of the workload's kernel to "
                         "profiles/ and exits")
    return ap.parse_args()


# ---------------------------------------------------------------- measured HBM traffic
# Per-launch HBM bytes of the dominant kernel come from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same
# counter reads for a plain copy of known size. The record is stored with a hash
# of the library sources; a bench run reports it only while the hash matches.
# kernels of the measured stage (per-launch traffic is the sum of their per-dispatch medians)
# (a name matches every kernel whose name holds it: both instances of the grouped GEMM)
PREFILL_KERNELS = ["prefill_count_kernel", "prefill_scatter_kernel", "expert_gemm_kernel<true,",
                   "expert_gemm_kernel<false,"]
FP8_KERNELS = ["prefill_count_kernel", "prefill_scatter_kernel", "quant_rows_fp8_kernel", "fp8_gemm_kernel<true>",
               "fp8_gemm_kernel<false>"]
# up to 8192 picks (1024 tokens at top-8) the dispatch has no count launch
TRAFFIC_KERNELS = {"decode": ["decode_layer_kernel"], "stack16": ["decode_layer_kernel"],
                   "stack1": ["decode_layer_kernel"],
                   "prefill512": PREFILL_KERNELS[1:], "prefill4096": PREFILL_KERNELS,
                   "prefill512_fp8": FP8_KERNELS[1:], "prefill4096_fp8": FP8_KERNELS,
                   "decode_8bit": ["decode_layer_kernel"], "prefill512_8bit": PREFILL_KERNELS[1:]}
# sources the measured kernels are built from: a stored traffic record holds for
# the sources it was taken on
DECODE_SOURCES = ["decode.hip", "route_device.h", "moe_internal.h", "abi.hip"]
PREFILL_SOURCES = ["prefill.hip", "prefill_internal.h", "mfma_common.h", "moe_internal.h", "abi.hip"]
FP8_SOURCES = ["prefill_fp8.hip", "prefill.hip", "prefill_internal.h", "mfma_common.h", "moe_internal.h"]
TRAFFIC_SOURCES = {"decode": DECODE_SOURCES, "stack16": DECODE_SOURCES, "stack1": DECODE_SOURCES,
                   "prefill512": PREFILL_SOURCES, "prefill4096": PREFILL_SOURCES,
                   "prefill512_fp8": FP8_SOURCES, "prefill4096_fp8": FP8_SOURCES,
                   "decode_8bit": DECODE_SOURCES, "prefill512_8bit": PREFILL_SOURCES}
ROOT = os.path.dirname(os.path.abspath(__file__))


def code_only(text):
    """C/C++ source without its comments, whitespace runs collapsed: what the traffic
    of a kernel can depend on (string and character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(wl):
    """Hash of the code (comments left out) of the sources the workload's measured
    kernels are built from, and of the headers."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_expert_fp32_amd", "csrc")
    for n in sorted(TRAFFIC_SOURCES[wl]):
        h.update(n.encode())
        h.update(code_only(open(os.path.join(csrc, n)).read()).encode())
    inc = os.path.join(ROOT, "include")
    for n in sorted(os.listdir(inc)):
        if n.endswith(".h"):
            h.update(n.encode())
            h.update(code_only(open(os.path.join(inc, n)).read()).encode())
    return h.hexdigest()[:16]


def traffic_path(wl):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % wl)


def pmc_values(folder, counter, name_part):
    """Per-dispatch values of one counter for kernels whose name contains name_part."""
    import csv

    out = {}
    for root, _, files in os.walk(folder):
        for f in files:
            if f.endswith("counter_collection.csv"):
                for r in csv.DictReader(open(os.path.join(root, f))):
                    if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                        key = (r["Dispatch_Id"], r["Kernel_Name"])
                        out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return list(out.values())


def write_traffic(wl, spec):
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = spec.split(",")
    kerns = TRAFFIC_KERNELS[wl]
    f = [pmc_values(fetch_dir, "FETCH_SIZE", k) for k in kerns]
    w = [pmc_values(write_dir, "WRITE_SIZE", k) for k in kerns]
    cal = json.load(open(os.path.join(cal_fetch_dir, "calibration.json")))
    known_kib = cal["bytes"] / 1024.0
    # the copy dispatches of the calibration run (ignore small set-up kernels)
    cf = [v for v in pmc_values(cal_fetch_dir, "FETCH_SIZE", "") if v > 0.5 * known_kib]
    cw = [v for v in pmc_values(cal_write_dir, "WRITE_SIZE", "") if v > 0.5 * known_kib]
    if not all(f) or not all(w) or not cf or not cw:
        raise SystemExit("missing counter values for %s" % kerns)
    k_fetch = known_kib / float(np.median(cf))
    k_write = known_kib / float(np.median(cw))
    # per launch: each kernel's dispatches summed over the run, divided by the number
    # of launches (the dispatch count of a kernel that runs once per launch; a kernel
    # such as the FP8 row quantiser runs twice)
    n_f = min(len(v) for v in f)
    n_w = min(len(v) for v in w)
    fk = sum(float(np.sum(v)) for v in f) / n_f
    wk = sum(float(np.sum(v)) for v in w) / n_w
    rec = {"workload": wl, "kernels": kerns, "dispatches": [[len(v) for v in f], [len(v) for v in w]],
           "fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
           "calibration_bytes": cal["bytes"], "fetch_scale": k_fetch, "write_scale": k_write,
           "traffic_bytes_per_launch": (fk * k_fetch + wk * k_write) * 1024.0,
           "source_hash": source_hash(wl)}
    os.makedirs(os.path.dirname(traffic_path(wl)), exist_ok=True)
    json.dump(rec, open(traffic_path(wl), "w"), indent=1)
    print(json.dumps(rec))


def stored_traffic(wl):
    try:
        rec = json.load(open(traffic_path(wl)))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(wl):
        log("stored traffic for %s predates the current sources: reported as null" % wl)
        return None
    return rec["traffic_bytes_per_launch"]


def copy_calibration(mib):
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    rec = {"bytes": n, "copies": 5}
    print(json.dumps(rec))
    return rec


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


WORKLOADS = ("decode", "prefill512", "prefill4096", "stack1", "stack16", "decode_8bit", "prefill512_8bit",
             "prefill512_fp8", "prefill4096_fp8")
METRIC = "MoE-layer tokens/s (decode bs1, prefill 512/4096) + % HBM/MFMA roofline"


class Inputs:
    """Device-resident layers and activations of one workload (the 40 stack layers
    are shared by stack1 and stack16)."""

    def __init__(self, wl, copies, cache):
        from quantized_moe_expert_fp32_amd import layer as L
        from quantized_moe_expert_fp32_amd import synth

        t0 = time.time()
        self.bits = 8 if wl.endswith("_8bit") else 4
        self.fp8 = wl.endswith("_fp8")
        wl = wl.replace("_8bit", "").replace("_fp8", "")
        if wl == "decode":
            base = synth.make_case("decode", bits=self.bits)
            self.hosts = [base.layers[0]] + [synth.make_layer(base.shape, base.seed, c) for c in range(1, copies)]
            self.x_host = np.concatenate([base.x, synth.random_x(base.seed, 63, 2048)], axis=0)
            self.T = 1
        elif wl in ("prefill512", "prefill4096"):
            base = synth.make_case(wl, bits=self.bits)
            self.hosts = [base.layers[0]]
            self.x_host = base.x
            self.T = base.T
        else:
            self.T = 1 if wl == "stack1" else 16
            base = synth.make_case("stack", T=self.T, n_layers=1)
            if "stack_hosts" not in cache:
                cache["stack_hosts"] = [base.layers[0]] + [synth.make_layer(base.shape, base.seed, l)
                                                           for l in range(1, 40)]
            self.hosts = cache["stack_hosts"]
            self.x_host = base.x
        self.shape = L.make_shape(base.shape)
        key = "stack_layers" if wl.startswith("stack") else "%s_%d%s_layers" % (wl, self.bits, "_fp8" * self.fp8)
        if key not in cache:
            # the prefill layout of the experts only where moe_experts_prefill reads it
            pf = not (wl.startswith("stack") or wl.startswith("decode") or self.fp8)
            cache[key] = [L.DeviceLayer(self.shape, h, fp8=self.fp8, prefill=pf) for h in self.hosts]
        self.layers = cache[key]
        self.x = L.to_device(self.x_host)
        # SHA-256 (first 16 hex digits) of the first layer's arrays and the activations
        self.sha256 = {k: v[:16] for k, v in self.hosts[0].sha256().items()}
        import hashlib

        self.sha256["x"] = hashlib.sha256(np.ascontiguousarray(self.x_host).tobytes()).hexdigest()[:16]
        self.setup_s = time.time() - t0


def run_workload(wl, K, W, inp, no_cpu, cpu_seconds):
    """Times K steps of one workload (graph replays) and its dominant stage; returns
    the record of the bench line for it."""
    import torch

    from quantized_moe_expert_fp32_amd import layer as L
    from quantized_moe_expert_fp32_amd import moe

    T, shape, layers, xs = inp.T, inp.shape, inp.layers, inp.x
    path = "fp8" if inp.fp8 else L.pick_path(T)
    kind = wl.replace("_8bit", "").replace("_fp8", "")
    buf = L.alloc_buffers(shape, T, path)
    S = shape.slots
    log("%s: %d weight sets, set-up %.1f s" % (wl, len(layers), inp.setup_s))

    # ---------------------------------------------------------------- the step sequence
    if kind.startswith("stack"):
        # one moe_decode_block (RMSNorm, layer, residual) per layer between two state
        # buffers; after the 40 layers the state is back in x_state
        x_state = xs.clone()
        x_other = torch.empty_like(x_state)
        period = 1

        def step(j):
            L.stack_step_fused(layers, x_state, x_other, buf)
    elif kind == "decode":
        period = xs.shape[0]  # 64 consecutive steps cover every token and every weight copy

        def step(j):
            dl = layers[j % len(layers)]
            r = j % period
            L.layer_step(dl, xs[r:r + 1], buf, path)
    else:
        period = 1

        def step(j):
            L.layer_step(layers[0], xs, buf, path)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for j in range(min(max(W, 1), 3)):
            step(j)
    torch.cuda.synchronize()

    # graphs: one of n_cap consecutive steps (n_cap = min(K, 64, a multiple of the
    # period)), replayed K // n_cap times, and one of the remaining K % n_cap steps
    n_cap = min(K, 64)
    if period > 1 and n_cap >= period:
        n_cap -= n_cap % period

    def capture(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(n):
                step(start + j)
        return g

    g_main = capture(n_cap, 0)
    rem = K % n_cap
    g_rem = capture(rem, (K // n_cap) * n_cap) if rem else None
    torch.cuda.synchronize()

    def run_steps(n):
        for _ in range(n // n_cap):
            g_main.replay()
        if n % n_cap:
            if n % n_cap == rem:
                g_rem.replay()
            else:
                with torch.cuda.stream(stream):
                    for j in range(n % n_cap):
                        step(j)

    with torch.cuda.stream(stream):
        run_steps(W)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev_a.record(stream)
        run_steps(K)
        ev_b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_us = ev_a.elapsed_time(ev_b) * 1e3
    value = T * K / elapsed
    log("%s: timed region %d steps in %.4f s (%.2f us per step on the stream)" % (wl, K, elapsed, region_us / K))

    # ---------------------------------------------------------------- dominant stage (HIP events on its stream)
    n_ev = min(max(K, 8), 512 if not kind.startswith("stack") else 200)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    if kind.startswith("stack"):
        # the stack's own launches: layer j % 40 on the state the previous layer left
        st_cur, st_nxt = xs.clone(), torch.empty_like(xs)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(200_000_000)  # keep the GPU busy while the host queues the measured launches
        for j in range(n_ev):
            dl = layers[j % len(layers)]
            xin = xs[(j % xs.shape[0]):(j % xs.shape[0]) + 1] if kind == "decode" else xs
            if kind.startswith("stack"):
                starts[j].record(stream)
                moe.moe_decode_block(shape, dl.router, dl.logit_bias, dl.experts, st_cur, T, 1e-6, buf.ws,
                                     buf.logits, buf.ids, buf.w, buf.wsh, buf.y, st_nxt)
                ends[j].record(stream)
                st_cur, st_nxt = st_nxt, st_cur
            elif path == "fused":
                starts[j].record(stream)
                moe.moe_decode_layer(shape, dl.router, dl.logit_bias, dl.experts, xin, T, buf.ws, buf.logits,
                                     buf.ids, buf.w, buf.wsh, buf.y, None, buf.out)
                ends[j].record(stream)
            else:
                moe.moe_route(shape, dl.router, dl.logit_bias, xin, T, buf.logits, buf.ids, buf.w, buf.wsh)
                starts[j].record(stream)
                if inp.fp8:
                    moe.moe_experts_prefill_fp8(shape, dl.experts_fp8, xin, T, buf.ids, buf.ws, buf.y)
                else:
                    moe.moe_experts_prefill(shape, dl.experts_prefill, xin, T, buf.ids, buf.ws, buf.y)
                ends[j].record(stream)
    torch.cuda.synchronize()
    durs_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    stage_us = float(np.mean(durs_ms) * 1e3)
    log("%s: dominant stage %.2f us average over %d event-timed launches" % (wl, stage_us, n_ev))
    if kind == "decode" or kind.startswith("stack"):
        # every step of the timed region is one decode_layer_kernel launch (the
        # stack: one per layer): the events around the graph-replayed region give
        # its average per-launch duration without the per-launch event overhead
        # of the eager launches above (2-3 us per launch)
        n_launch = K * (len(layers) if kind.startswith("stack") else 1)
        stage_us = region_us / n_launch
        log("%s: decode_layer_kernel %.2f us per launch over the timed region" % (wl, stage_us))

    # algorithmic work of one launch of the dominant stage: the weights of every
    # distinct expert it touches (read once) plus the activations; the fp32 slot
    # buffer and the bf16 intermediate are not counted
    ids_np = buf.ids.cpu().numpy()
    distinct = len(set(ids_np.reshape(-1).tolist())) + shape.has_shared
    if kind.startswith("stack"):
        # the stack's tokens drift together layer by layer and share more experts
        # than the first layer's: the mean over one pass of the 40 layers
        keep = []
        with torch.cuda.stream(stream):
            L.stack_step_fused(layers, xs.clone(), torch.empty_like(xs), buf, keep=keep)
        torch.cuda.synchronize()
        distinct = float(np.mean([len(set(ids.cpu().numpy().reshape(-1).tolist())) for _, ids in keep]))
        distinct += shape.has_shared
    per_expert = FP8_EXPERT_BYTES if inp.fp8 else EXPERT_BYTES_8BIT if inp.bits == 8 else EXPERT_BYTES
    alg_bytes = int(distinct * per_expert) + T * 2048 * 2
    flops = T * S * 3 * 2 * 2048 * 512
    if path == "fused":
        alg_bytes += ROUTER_BYTES  # the launch also streams the router
    if inp.fp8:
        # the FP8 weights (1 byte per weight) take longer to stream at 8 TB/s than the
        # FP8 products take at 5 PFLOP/s, at 512 and at 4096 tokens alike
        roof = dict(bound="hbm", achieved=alg_bytes / (stage_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
        roof["mfma_fp8_frac"] = flops / (stage_us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS
    elif wl == "prefill4096":
        roof = dict(bound="mfma", achieved=flops / (stage_us * 1e-6) / 1e12, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=alg_bytes / (stage_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(wl)
    roof["kernel"] = ("decode_layer_kernel (RMSNorm, router, selection, experts, combine and residual in one launch)"
                      if kind.startswith("stack") else
                      "decode_layer_kernel (router, selection, experts, combine in one launch)" if path == "fused"
                      else "experts stage (moe_experts_prefill_fp8): " + " + ".join(TRAFFIC_KERNELS[wl]) if inp.fp8
                      else "experts stage (moe_experts_prefill): " + " + ".join(k.rstrip(",") + ", …>" if k.endswith(",") else k
                                                                     for k in TRAFFIC_KERNELS[wl]))
    roof["avg_us"] = stage_us
    roof["alg_bytes_per_launch"] = int(alg_bytes)
    roof["alg_flops_per_launch"] = int(flops)

    cpu = None
    if not no_cpu:
        cpu = cpu_baseline(kind, inp.hosts, inp.x_host, T, shape, cpu_seconds, fp8=inp.fp8)
    unit = "layer-tokens/s" if not kind.startswith("stack") else "tokens/s"
    return {
        "value": value, "unit": unit, "steps": K, "warmup": W, "ms_per_step": elapsed * 1e3 / K,
        "us_per_step_stream": region_us / K,
        "config": {"workload": wl, "T": T, "hidden": 2048, "n_experts": 256, "top_k": 8, "shared": 1,
                   "inter": 512, "weights": ("E4M3 rows upcast from int%d affine g64" if inp.fp8 else
                                             "int%d affine g64") % inp.bits, "router": "8-bit affine g64",
                   "layers": len(layers) if kind.startswith("stack") else 1,
                   "weight_copies": len(layers) if kind == "decode" else 1, "path": path,
                   "graph_steps": n_cap},
        "roofline": roof, "cpu_baseline": cpu, "inputs_sha256": inp.sha256, "setup_s": inp.setup_s,
    }


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.workload, args.traffic_from)
        return
    if args.copy_calibration:
        rec = copy_calibration(args.copy_calibration)
        out = os.environ.get("CALIBRATION_OUT")
        if out:
            os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
            json.dump(rec, open(out, "w"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert parallelism "
              "across GPUs is not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(torch.device("cuda:0"))
    head = args.workload
    defaults = {"decode": (2048, 256), "prefill512": (200, 20), "prefill4096": (50, 5),
                "stack1": (50, 5), "stack16": (50, 5), "decode_8bit": (1024, 128), "prefill512_8bit": (100, 10),
                "prefill512_fp8": (200, 20), "prefill4096_fp8": (50, 5)}
    K = args.steps if args.steps is not None else defaults[head][0]
    W = args.warmup if args.warmup is not None else defaults[head][1]
    cache = {}
    rec = run_workload(head, K, W, Inputs(head, args.copies, cache), args.no_cpu_baseline, args.cpu_seconds)
    others = {}
    if not args.only:
        # the other configurations of the metric, each with its own roofline; the
        # step and warm-up counts are the headline's, capped by the workload's default
        for wl in WORKLOADS:
            if wl == head:
                continue
            k2 = min(K, defaults[wl][0])
            w2 = min(W, defaults[wl][1])
            r = run_workload(wl, k2, w2, Inputs(wl, args.copies, cache), args.no_cpu_baseline,
                             min(args.cpu_seconds, 5.0))
            for drop in ("setup_s",):
                r.pop(drop, None)
            others[wl] = r
            for key in [k2_ for k2_ in cache if k2_.startswith(wl.replace("_8bit", "").replace("_fp8", ""))
                        and k2_.endswith("_layers")]:
                cache.pop(key, None)  # free what no later workload reads
    line = {
        "metric": METRIC, "value": rec["value"], "unit": rec["unit"], "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 activations, int4 weights, fp32/fp64 accumulation", "data": "synthetic",
        "config": rec["config"], "roofline": rec["roofline"], "cpu_baseline": rec["cpu_baseline"],
        "inputs_sha256": rec["inputs_sha256"], "us_per_step_stream": rec["us_per_step_stream"],
        "setup_s": rec["setup_s"], "workloads": others,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, hosts, xs_host, T, shape, budget_s, fp8=False):
    """The FP64 oracle as it stands, on a bounded sample of the same workload (fp8:
    the oracle's FP8 route)."""
    from oracle import moe_oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    k = shape.top_k
    t0 = time.perf_counter()
    done_tokens = 0
    layer_passes = 0
    if wl == "decode":
        j = 0
        while time.perf_counter() - t0 < budget_s and j < 256:
            O.layer_forward(xs_host[j % len(xs_host)][None, :], hosts[j % len(hosts)], k)
            done_tokens += 1
            j += 1
        sample = "%d single-token layer passes over the rotating copies/tokens" % done_tokens
    elif wl.startswith("prefill"):
        n = min(T, 64)
        while time.perf_counter() - t0 < budget_s and layer_passes < 4:
            O.layer_forward(xs_host[:n], hosts[0], k, fp8=fp8)
            done_tokens += n
            layer_passes += 1
        sample = "%d passes of the first %d tokens through the layer%s" % (layer_passes, n,
                                                                          " (FP8 route)" if fp8 else "")
    else:
        n = xs_host.shape[0]
        x = xs_host
        for l in range(len(hosts)):
            if layer_passes and time.perf_counter() - t0 >= budget_s:
                break
            x = O.residual_bf16(x, O.layer_forward(O.rmsnorm_bf16(x), hosts[l], k)["out"])
            layer_passes += 1
        done_tokens = n * layer_passes
        sample = "%d tokens through the first %d of the 40 layers (layer-tokens)" % (n, layer_passes)
    el = time.perf_counter() - t0
    return {"value": done_tokens / el, "unit": "layer-tokens/s", "cores": cores, "host_cores": os.cpu_count(),
            "kind": "oracle", "sample": sample, "seconds": el}


if __name__ == "__main__":
    main()
