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
  stack1/16    one decode step of T=1 / T=16 tokens through 40 stacked layers.
The timed region replays HIP graphs of the step sequence (captured once).
Rank 0 prints one JSON line; `roofline` covers the expert stage (the kernels
launched by moe_experts_decode / moe_experts_prefill), timed with HIP events
on the launch stream; `cpu_baseline` times the FP64 oracle on a bounded sample.
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
ROUTER_BYTES = 559_232


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill512", "prefill4096", "stack1", "stack16"])
    ap.add_argument("--copies", type=int, default=8, help="independent weight sets for the decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
PREFILL_KERNELS = ["prefill_count_kernel", "prefill_scatter_kernel", "expert_gemm_kernel<true>",
                   "expert_gemm_kernel<false>"]
TRAFFIC_KERNELS = {"decode": ["decode_layer_kernel"], "stack16": ["decode_layer_kernel"],
                   "stack1": ["decode_layer_kernel"],
                   "prefill512": PREFILL_KERNELS, "prefill4096": PREFILL_KERNELS}
# sources the measured kernels are built from: a stored traffic record holds for
# the sources it was taken on
DECODE_SOURCES = ["decode.hip", "route_device.h", "moe_internal.h", "abi.hip"]
PREFILL_SOURCES = ["prefill.hip", "mfma_common.h", "moe_internal.h", "abi.hip"]
TRAFFIC_SOURCES = {"decode": DECODE_SOURCES, "stack16": DECODE_SOURCES, "stack1": DECODE_SOURCES,
                   "prefill512": PREFILL_SOURCES, "prefill4096": PREFILL_SOURCES}
ROOT = os.path.dirname(os.path.abspath(__file__))


def source_hash(wl):
    """Hash of the sources the workload's measured kernels are built from (and the headers)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_expert_fp32_amd", "csrc")
    for n in sorted(TRAFFIC_SOURCES[wl]):
        h.update(n.encode())
        h.update(open(os.path.join(csrc, n), "rb").read())
    inc = os.path.join(ROOT, "include")
    for n in sorted(os.listdir(inc)):
        if n.endswith(".h"):
            h.update(n.encode())
            h.update(open(os.path.join(inc, n), "rb").read())
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
    fk = sum(float(np.median(v)) for v in f)
    wk = sum(float(np.median(v)) for v in w)
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


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.workload, args.traffic_from)
        return
    if args.copy_calibration:
        rec = copy_calibration(args.copy_calibration)
        out = os.environ.get("CALIBRATION_OUT")
        if out:
            json.dump(rec, open(out, "w"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert parallelism "
              "is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_moe_expert_fp32_amd import layer as L
    from quantized_moe_expert_fp32_amd import moe, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = args.workload
    defaults = {"decode": (2048, 256), "prefill512": (200, 20), "prefill4096": (50, 5),
                "stack1": (50, 5), "stack16": (50, 5)}
    K = args.steps if args.steps is not None else defaults[wl][0]
    W = args.warmup if args.warmup is not None else defaults[wl][1]

    # ---------------------------------------------------------------- inputs
    t_setup = time.time()
    if wl == "decode":
        base = synth.make_case("decode")
        shape = L.make_shape(base.shape)
        hosts = [base.layers[0]] + [synth.make_layer(base.shape, base.seed, c) for c in range(1, args.copies)]
        layers = [L.DeviceLayer(shape, h) for h in hosts]
        NX = 64
        xs_host = np.concatenate([base.x, synth.random_x(base.seed, NX - 1, 2048)], axis=0)
        T = 1
    elif wl in ("prefill512", "prefill4096"):
        base = synth.make_case(wl)
        shape = L.make_shape(base.shape)
        hosts = [base.layers[0]]
        layers = [L.DeviceLayer(shape, hosts[0])]
        xs_host = base.x
        T = base.T
    else:
        T = 1 if wl == "stack1" else 16
        base = synth.make_case("stack", T=T, n_layers=1)
        shape = L.make_shape(base.shape)
        hosts = [base.layers[0]]
        layers = [L.DeviceLayer(shape, hosts[0])]
        for l in range(1, 40):
            layers.append(L.DeviceLayer(shape, synth.make_layer(base.shape, base.seed, l)))
        xs_host = base.x
    setup_s = time.time() - t_setup
    log("setup done in %.1f s (%s, %d weight sets)" % (setup_s, wl, len(layers)))
    path = L.pick_path(T)
    xs = L.to_device(xs_host)
    buf = L.alloc_buffers(shape, T, path)
    S = shape.slots

    # ---------------------------------------------------------------- the step sequence
    if wl.startswith("stack"):
        x_state = xs.clone()
        xn = torch.empty_like(x_state)
        seq_len = 1

        def step(j):
            L.stack_step(layers, x_state, xn, buf, path=path)
    elif wl == "decode":
        seq_len = NX  # one graph covers 64 consecutive steps (every token, every copy)

        def step(j):
            dl = layers[j % len(layers)]
            r = j % NX
            L.layer_step(dl, xs[r:r + 1], buf, path)
    else:
        seq_len = 1

        def step(j):
            L.layer_step(layers[0], xs, buf, path)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for j in range(min(W, 3)):
            step(j)
    torch.cuda.synchronize()

    # graphs of seq_len consecutive steps; replay g covers steps g*seq_len .. +seq_len
    graphs = []
    for gi in range(1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(seq_len):
                step(gi * seq_len + j)
        graphs.append(g)
    torch.cuda.synchronize()

    def run_steps(n, start=0):
        done = 0
        gi = 0
        while done + seq_len <= n:
            graphs[gi % len(graphs)].replay()
            gi += 1
            done += seq_len
        if done < n:
            with torch.cuda.stream(stream):
                for j in range(done, n):
                    step(start + j)

    with torch.cuda.stream(stream):
        run_steps(W)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    torch.cuda.synchronize()
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev_a.record(stream)
        run_steps(K)
        ev_b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_us = ev_a.elapsed_time(ev_b) * 1e3
    ms_per_step = elapsed * 1e3 / K
    tokens_per_step = T
    value = tokens_per_step * K / elapsed
    log("timed region: %d steps in %.3f s" % (K, elapsed))

    # ---------------------------------------------------------------- expert-stage timing (HIP events)
    n_ev = min(K, 512)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    with torch.cuda.stream(stream):
        torch.cuda._sleep(200_000_000)  # keep the GPU busy while the host queues the measured launches
        for j in range(n_ev):
            dl = layers[j % len(layers)]
            xin = xs[(j % xs.shape[0]):(j % xs.shape[0]) + 1] if wl == "decode" else xs
            if path == "fused":
                # the whole decode layer is one kernel (decode_layer_kernel)
                starts[j].record(stream)
                moe.moe_decode_layer(shape, dl.router, dl.logit_bias, dl.experts, xin, T, buf.ws, buf.logits, buf.ids,
                                     buf.w, buf.wsh, buf.y, None, buf.out)
                ends[j].record(stream)
            else:
                moe.moe_route(shape, dl.router, dl.logit_bias, xin, T, buf.logits, buf.ids, buf.w, buf.wsh)
                starts[j].record(stream)
                moe.moe_experts_prefill(shape, dl.experts, xin, T, buf.ids, buf.ws, buf.y)
                ends[j].record(stream)
    torch.cuda.synchronize()
    durs_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    expert_us = float(np.mean(durs_ms) * 1e3)
    log("measured stage: %.2f us average over %d event-timed launches" % (expert_us, n_ev))
    if wl == "decode":
        # every step of the timed region is exactly one decode_layer_kernel launch:
        # the events around the region give the kernel's average duration without
        # the per-launch event overhead
        expert_us = region_us / K
        log("decode_layer_kernel: %.2f us average over the %d launches of the timed region" % (expert_us, K))

    # algorithmic work of one expert-stage launch
    ids_np = buf.ids.cpu().numpy()
    # (weights of every distinct expert the launch touches, read once, plus the activations;
    # the fp32 slot buffer and the bf16 intermediate are not counted)
    distinct = len(set(ids_np.reshape(-1).tolist())) + shape.has_shared
    alg_bytes = distinct * EXPERT_BYTES + T * 2048 * 2
    flops = T * S * 3 * 2 * 2048 * 512
    if path == "fused":
        alg_bytes += ROUTER_BYTES  # the launch also streams the router
    if path in ("decode", "fused"):
        roof = dict(bound="hbm", achieved=alg_bytes / (expert_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        if wl == "prefill4096":
            roof = dict(bound="mfma", achieved=flops / (expert_us * 1e-6) / 1e12, peak=BF16_PEAK_TFLOPS,
                        unit="TFLOP/s")
        else:
            roof = dict(bound="hbm", achieved=alg_bytes / (expert_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS,
                        unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(wl)
    roof["kernel"] = ("decode_layer_kernel (router, selection, experts, combine in one launch)" if path == "fused"
                      else "experts stage (moe_experts_prefill): " + " + ".join(PREFILL_KERNELS))
    roof["avg_us"] = expert_us
    roof["alg_bytes_per_launch"] = int(alg_bytes)

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, hosts, xs_host, T, shape, args.cpu_seconds)

    unit = "layer-tokens/s" if not wl.startswith("stack") else "tokens/s"
    metric = "MoE-layer tokens/s (decode bs1, prefill 512/4096) + % HBM/MFMA roofline"
    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 activations, int4 weights, fp32/fp64 accumulation", "data": "synthetic",
        "config": {"workload": wl, "T": T, "hidden": 2048, "n_experts": 256, "top_k": 8, "shared": 1,
                   "inter": 512, "weights": "int4 affine g64", "router": "8-bit affine g64",
                   "layers": len(layers) if wl.startswith("stack") else 1,
                   "weight_copies": len(layers) if wl == "decode" else 1, "path": path},
        "roofline": roof,
        "cpu_baseline": cpu,
        "setup_s": setup_s,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, hosts, xs_host, T, shape, budget_s):
    """The FP64 oracle as it stands, on a bounded sample of the same workload."""
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
        unit = "layer-tokens/s"
    elif wl.startswith("prefill"):
        n = min(T, 64)
        while time.perf_counter() - t0 < budget_s and layer_passes < 4:
            O.layer_forward(xs_host[:n], hosts[0], k)
            done_tokens += n
            layer_passes += 1
        sample = "%d passes of the first %d tokens through the layer" % (layer_passes, n)
        unit = "layer-tokens/s"
    else:
        n = xs_host.shape[0]
        x = xs_host
        for l in range(len(hosts)):
            x = O.residual_bf16(x, O.layer_forward(O.rmsnorm_bf16(x), hosts[l], k)["out"])
            layer_passes += 1
        done_tokens = n * layer_passes
        sample = "%d tokens through %d of the 40 layers (layer-tokens)" % (n, layer_passes)
        unit = "layer-tokens/s"
    el = time.perf_counter() - t0
    return {"value": done_tokens / el, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample,
            "seconds": el}


if __name__ == "__main__":
    main()
