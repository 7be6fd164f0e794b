"""Throughput of the sparse MoE layer on one MI355X, with its roofline and the CPU oracle beside it.

Default workload (decode, A3B-like shape): hidden 2048, 128 NVFP4 experts,
top-8 renormalised, SwiGLU intermediate 768, Zipf(1.1) router logits.  One
step = one layer call at each of the batch sizes 1, 4 and 16 tokens (21
tokens).  Every step uses a fresh seeded batch and the next of 8 HBM copies
of the layer's experts, so no expert is served from the 256 MB last-level
cache across steps.  Inputs are resident in HBM before timing starts.

Other workloads (--workload):
  prefill-mxfp4  4096 tokens, MXFP4 weights x MXFP4 activations (FP4 matrix cores)
  prefill-bf16   4096 tokens, BF16 weights (bf16 matrix cores)
  large-decode   hidden 7168, 256 + 1 shared MXFP4 experts, intermediate 2048, 1 token
  large-prefill  the same layer, 2048 tokens, MXFP4 activations
  stream         cached decode: 48 A3B-like NVFP4 layers in a pinned host bank,
                 2048 HBM slots under LRU, 512 single-token steps from a cold
                 cache; misses copied host->device on a side stream

Prints one JSON line (see the design doc for the definitions of every field).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "bf16": 2500.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def moe_w13_bytes(fmt, H, I):
    """Packed gate + up weights and scales of one expert (E2M1 + E8M0 per 32,
    E2M1 + E4M3 per 16 + per-tensor fp32 scales, or bf16)."""
    n = 2 * H * I
    if fmt == "bf16":
        return 2 * n
    if fmt == "mxfp4":
        return n // 2 + n // 32
    return n // 2 + n // 16 + 8


def measured_traffic(workload, root):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or
    None when there is none or its kernel sources have changed since."""
    import hashlib
    path = os.path.join(root, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    h = hashlib.sha256()
    for src in t.get("sources", []):
        with open(os.path.join(root, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != t.get("sources_sha256"):
        return None
    return t.get("bytes_per_launch")


class Timer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((s, e))

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs)

    def reset(self):
        self.pairs = []


def oracle_baseline(run_one, unit_count, budget_s=12.0):
    """Time the oracle (as it stands) on a bounded sample; returns (value per second, sample count, threads)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    n = 0
    while True:
        run_one(n)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return n * unit_count / dt, n, threads, dt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill-mxfp4", "prefill-bf16", "large-decode", "large-prefill", "stream"])
    ap.add_argument("--copies", type=int, default=8, help="HBM copies of the layer's experts cycled across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--stream-tokens", type=int, default=512, help="tokens of the stream workload")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="first run three plain device copies of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="no GPU work: 'stats CSV OUT CMD' writes a kernel-time summary; "
                         "'traffic FETCH_CSV WRITE_CSV COPY_MIB OUT CMD' writes the dominant kernel's HBM bytes")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md, 'How the path would shard').", file=sys.stderr)
        sys.exit(2)

    if args.workload == "stream":
        return bench_stream(args)

    import torch

    import synth
    from fp4_expert_ffn_amd.layer import MoELayer, bf16_tensor, blob_of

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    wl = args.workload

    if wl == "decode":
        cfg = synth.A3B
        fmt, amode, batches, shared = "nvfp4", "bf16", [1, 4, 16], False
        make = lambda: synth.a3b_experts("nvfp4", config=1)
        steps, warmup = args.steps or 300, args.warmup or 30
        nb = 64
        inputs = [[synth.decode_batch(T, i) for T in batches] for i in range(nb)]
    elif wl.startswith("prefill"):
        cfg = synth.A3B
        fmt = "mxfp4" if wl == "prefill-mxfp4" else "bf16"
        amode, batches, shared = fmt, [4096], False
        make = lambda: synth.a3b_experts(fmt, config=2)
        steps, warmup = args.steps or 30, args.warmup or 5
        nb = 1
        inputs = [[synth.prefill_batch(4096)]]
    else:
        cfg = synth.LARGE
        fmt, shared = "mxfp4", True
        T = 1 if wl == "large-decode" else 2048
        amode = "bf16" if T == 1 else "mxfp4"
        batches = [T]
        make = None
        steps, warmup = args.steps or (200 if T == 1 else 10), args.warmup or (20 if T == 1 else 3)
        nb = 1
        inputs = [[synth.large_batch(T)]]
        args.copies = 1 if T > 1 else min(args.copies, 4)

    E, k, H, I = cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    Tmax = max(batches)
    if wl.startswith("prefill"):
        args.copies = min(args.copies, 2)
    log(f"[bench] workload={wl}: generating experts")
    t0 = time.perf_counter()
    if make is not None:
        experts = make()
        shared_ex = None
    else:
        experts = [synth.large_expert(e) for e in range(E)]
        shared_ex = synth.large_expert(synth.SHARED_EXPERT)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f}s; uploading {args.copies} copies")
    layers = []
    blobs = [blob_of(ex) for ex in experts]
    shared_blob = blob_of(shared_ex) if shared_ex is not None else None
    for c in range(args.copies):
        lay = MoELayer(E=E, k=k, H=H, I=I, fmt=fmt, max_tokens=Tmax, device=dev, shared=shared, amode=amode)
        for e, b in enumerate(blobs):
            lay.load_expert(e, b)
        if shared:
            lay.load_shared(shared_blob)
        layers.append(lay)
    blob_bytes = layers[0].blob_bytes
    del blobs

    if args.calibration_copy:
        n = args.calibration_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # one elementwise kernel: reads and writes MIB MiB
        torch.cuda.synchronize()
        del src, dst

    # One "combo" per input batch group: its own routing/output buffers, weights copy i % copies.
    combos = []
    for i, group in enumerate(inputs):
        lay = layers[i % len(layers)]
        calls = []
        for b in group:
            T = b["x"].shape[0]
            x = bf16_tensor(b["x"], dev)
            lg = torch.from_numpy(b["logits"]).to(dev) if "logits" in b else None
            wr = torch.from_numpy(b["w_router"]).to(dev) if "w_router" in b else None
            st = lay.new_state(T)
            calls.append((T, x, lg, wr, st, st.args(T, x)))
        combos.append(calls)
    n_per_graph = len(combos)
    toks_per_step = sum(c[0] for c in combos[0])

    def run_full():
        for calls in combos:
            for (T, x, lg, wr, st, a) in calls:
                st.route(T, x=x, w_router=wr, logits=lg)
                st.ffn(T, x, args=a)

    # eager pass (library set-up, workspace sizing), then capture the sequence as a HIP graph
    run_full()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g_full = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_full, stream=side):
        run_full()
    torch.cuda.synchronize()

    replays = max(1, -(-steps // n_per_graph))
    steps = replays * n_per_graph
    wreps = max(1, -(-warmup // n_per_graph))
    warmup = wreps * n_per_graph
    log(f"[bench] warmup {warmup} steps, timing {steps} steps ({replays} graph replays of {n_per_graph} steps)")
    for _ in range(wreps):
        g_full.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(replays):
        g_full.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    value = toks_per_step * steps / wall

    # Dominant kernel (the gate/up projection): its launch durations from HIP
    # events recorded at the kernel's own start and end (moe_expert_ffn_traced),
    # over the same calls run eagerly, the same number of steps.  Launch order:
    # GEMV path gate/up, down, combine; FP4 path quantiser, gate/up, down,
    # combine; BF16 matrix-core path gate/up, down, combine.
    from fp4_expert_ffn_amd import moe_expert_ffn_traced
    dom = 1 if amode == "mxfp4" else 0
    stream_now = torch.cuda.current_stream()
    # The calls are enqueued in batches behind a short spin kernel on the same
    # stream, so the GPU never waits for the host inside a timed launch (an
    # eager launch sequence is host-bound, and an idle gap between an event
    # and its kernel would count as kernel time).
    flat = [c for _ in range(replays) for calls in combos for c in calls]
    clock_hz = torch.cuda.get_device_properties(0).clock_rate * 1e3 if hasattr(
        torch.cuda.get_device_properties(0), "clock_rate") else 2.4e9
    pairs = []
    batch = 16
    for i in range(0, len(flat), batch):
        torch.cuda._sleep(int(0.012 * clock_hz))  # about 12 ms of backlog
        for (T, x, lg, wr, st, a) in flat[i:i + batch]:
            st.route(T, x=x, w_router=wr, logits=lg)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
            for e in evs:
                e.record(stream_now)  # creates the HIP events; re-recorded by the launches
            n = moe_expert_ffn_traced(a, evs)
            assert n >= 2 * (dom + 1), n
            pairs.append((evs[2 * dom], evs[2 * dom + 1]))
    torch.cuda.synchronize()
    durs = [e0.elapsed_time(e1) for e0, e1 in pairs]
    dom_ms = sum(durs) / len(durs)

    # algorithmic bytes / flops of the dominant kernel (gate/up projection + SwiGLU),
    # per launch, from the routing each call holds
    w13_bytes = moe_w13_bytes(fmt, H, I)
    tot_bytes, tot_flops, n_calls = 0, 0.0, 0
    for calls in combos:
        for (T, x, lg, wr, st, a) in calls:
            cn = st.counts.cpu().numpy()
            rows = int(np.sum(cn)) + (T if shared else 0)
            active = int(np.count_nonzero(cn)) + (1 if shared else 0)
            act = 2 if amode == "bf16" else 0.53125  # bf16, or MXFP4 codes + E8M0 per 32, per value
            tot_bytes += active * w13_bytes + T * H * act + rows * I * act
            tot_flops += 2.0 * rows * 2 * I * H
            n_calls += 1
    bytes_per_launch = tot_bytes / n_calls
    flops_per_launch = tot_flops / n_calls
    kname = {"bf16": "k_gemv (gate/up projection + SwiGLU, bf16 operands)",
             "mxfp4": "k_fp4_gemm<0, true> (gate/up projection + SwiGLU, FP4 matrix cores)"}[amode]
    if wl.startswith("prefill-bf16"):
        kname = "k_fp4_gemm<0, false> (gate/up projection + SwiGLU, bf16 weights on bf16 matrix cores)"
    elif fmt == "nvfp4":
        kname = "k_gemv (gate/up projection + SwiGLU, NVFP4 weights on fp16 matrix cores)"
    # The large-expert prefill sits below the FP4 ridge (about 267 FLOP/B): HBM bounds it.
    if amode == "mxfp4" and wl != "large-prefill":
        ach = flops_per_launch / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS["fp4"], "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK_TFLOPS["fp4"], 4)}
        roof["hbm_gbs_same_kernel"] = round(bytes_per_launch / (dom_ms * 1e-3) / 1e9, 1)
    else:
        ach = bytes_per_launch / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
        if fmt == "bf16":
            roof["bf16_mfma_tflops_same_kernel"] = round(flops_per_launch / (dom_ms * 1e-3) / 1e12, 1)
        if amode == "mxfp4":
            roof["fp4_mfma_tflops_same_kernel"] = round(flops_per_launch / (dom_ms * 1e-3) / 1e12, 1)
    roof["traffic"] = measured_traffic(wl, ROOT)
    roof["kernel"] = kname
    roof["avg_launch_us"] = round(dom_ms * 1e3, 3)
    roof["launches_averaged"] = len(durs)
    roof["algorithmic_bytes_per_launch"] = int(bytes_per_launch)
    roof["algorithmic_flops_per_launch"] = int(flops_per_launch)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] timing the CPU oracle on a bounded sample")
        b0 = inputs[0]
        sample_tokens = sum(b["x"].shape[0] for b in b0)
        if wl == "decode" or wl == "large-decode":
            def run_one(n):
                for b in inputs[n % len(inputs)]:
                    if "logits" in b:
                        oracle.moe.layer(b["x"], experts, k, logits=b["logits"])
                    else:
                        oracle.moe.layer(b["x"], experts, k, w_router=b["w_router"], shared=shared_ex)
            val, n, thr, dt = oracle_baseline(run_one, sample_tokens, args.cpu_budget)
            cpu = {"value": round(val, 3), "unit": "tokens/s", "cores": thr, "kind": "oracle",
                   "sample": f"{n} oracle layer calls over batches of {[b['x'].shape[0] for b in b0]} tokens "
                             f"({dt:.1f} s)"}
        else:
            b = b0[0]
            ids, w = oracle.moe.route(b["logits"], k) if "logits" in b else (None, None)
            if ids is None:
                ids, w = oracle.moe.route(combos[0][0][4].logits[:b["x"].shape[0]].cpu().numpy(), k)
            cache = {}

            def wts(e):
                if e not in cache:
                    cache.clear()
                    cache[e] = oracle.moe.dequant_expert(experts[e])
                return cache[e]
            rng = np.random.default_rng(0)
            order = rng.permutation(b["x"].shape[0])
            sw = oracle.moe.dequant_expert(shared_ex) if shared_ex is not None else None

            def run_one(n):
                t = int(order[n % len(order)])
                oracle.moe.token_output(t, b["x"], ids[t], w[t], wts, shared_weights=sw, amode=amode)
            val, n, thr, dt = oracle_baseline(run_one, 1, args.cpu_budget)
            cpu = {"value": round(val, 3), "unit": "tokens/s", "cores": thr, "kind": "oracle",
                   "sample": f"{n} tokens of the {b['x'].shape[0]}-token batch, one by one ({dt:.1f} s)"}

    names = {"decode": "decode A3B-like NVFP4 (hidden 2048, 128 experts, top-8, inter 768), batches 1+4+16",
             "prefill-mxfp4": "prefill A3B-like 4096 tokens, MXFP4 weights x MXFP4 activations",
             "prefill-bf16": "prefill A3B-like 4096 tokens, BF16 weights",
             "large-decode": "large-expert layer (hidden 7168, 256+1 shared MXFP4 experts, inter 2048), 1 token",
             "large-prefill": "large-expert layer, 2048 tokens, MXFP4 activations"}
    line = {
        "metric": "MoE-layer tokens/s",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"decode": "nvfp4xbf16->f32", "prefill-mxfp4": "mxfp4xmxfp4->f32", "prefill-bf16": "bf16->f32",
                  "large-decode": "mxfp4xbf16->f32", "large-prefill": "mxfp4xmxfp4->f32"}[wl],
        "data": "synthetic (seeded; weights N(0,0.02) quantised, activations N(0,1) bf16, Zipf(1.1) routing)",
        "config": {"workload": names[wl], "tokens_per_step": toks_per_step, "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "weights": fmt, "hbm_copies": len(layers),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer_ms_per_call": round(wall / (replays * n_calls) * 1e3, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


# Kernel-name patterns of the dominant kernel (gate/up projection) per workload.
DOMINANT = {"decode": "k_gemv<2, false", "large-decode": "k_gemv<1, false", "prefill-mxfp4": "k_fp4_gemm<0, true>",
            "large-prefill": "k_fp4_gemm<0, true>", "prefill-bf16": "k_fp4_gemm<0, false>"}
KERNEL_SOURCES = ["fp4_expert_ffn_amd/csrc/ffn_gemv.hip", "fp4_expert_ffn_amd/csrc/ffn_mfma.hip",
                  "fp4_expert_ffn_amd/csrc/ffn_fp4gemm.hip", "fp4_expert_ffn_amd/csrc/ffn_common.h",
                  "fp4_expert_ffn_amd/csrc/common.h"]


def _pmc_rows(path, counter):
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def summarize(args):
    """Text summaries of rocprofv3 output for profiles/ (runs no GPU work)."""
    import csv
    import hashlib
    kind = args.summarize[0]
    if kind == "stats":
        src, out, cmd = args.summarize[1:4]
        with open(src) as f:
            rows = list(csv.DictReader(f))
        lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}", "",
                 f"{'kernel':<90} {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
        for r in rows[:12]:
            lines.append(f"{r['Name'][:90]:<90} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>10.2f} "
                         f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                         f"{float(r['Percentage']):>6.2f}")
        # the dominant kernel over all its instantiations (a call-weighted average)
        wl = os.path.basename(out)[len("kernels_"):-len(".txt")]
        pat = DOMINANT.get(wl)
        dom = [r for r in rows if pat and pat in r["Name"]]
        if dom:
            calls = sum(int(r["Calls"]) for r in dom)
            tot = sum(float(r["TotalDurationNs"]) for r in dom)
            lines += ["", f"dominant kernel '{pat}' ({len(dom)} instantiations): {calls} calls, "
                          f"average {tot / calls / 1e3:.2f} us"]
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote {out}")
        return
    if kind == "traffic":
        fetch_csv, write_csv, copy_mib, out, cmd = args.summarize[1:6]
        wl = os.path.basename(out)[len("traffic_"):-len(".json")]
        pat = DOMINANT[wl]
        copy_bytes = int(copy_mib) << 20
        res = {}
        for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
            rows = _pmc_rows(path, name)
            cal = [v for k, v in rows if "neg" in k][:3]
            dom = [v for k, v in rows if pat in k]
            if not cal or not dom:
                raise SystemExit(f"{name}: no calibration copy or no {pat} dispatch in {path}")
            res[name] = {"kib_per_dispatch": sum(dom) / len(dom), "dispatches": len(dom),
                         "copy_kib": sum(cal) / len(cal), "bytes_per_kib": copy_bytes / (sum(cal) / len(cal))}
        h = hashlib.sha256()
        for src in KERNEL_SOURCES:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        fetch = res["FETCH_SIZE"]["kib_per_dispatch"] * res["FETCH_SIZE"]["bytes_per_kib"]
        write = res["WRITE_SIZE"]["kib_per_dispatch"] * res["WRITE_SIZE"]["bytes_per_kib"]
        t = {"workload": wl, "kernel_pattern": pat, "command": cmd, "counters": res,
             "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
             "bytes_per_launch": int(fetch + write), "copy_bytes": copy_bytes,
             "sources": KERNEL_SOURCES, "sources_sha256": h.hexdigest()}
        with open(out, "w") as f:
            json.dump(t, f, indent=1)
        print(f"wrote {out}: {int(fetch + write)} bytes per launch")
        return
    raise SystemExit(f"unknown summary kind {kind}")


def bench_stream(args):
    """Cached decode stream: tokens/s of 512 single-token steps through 48 layers."""
    import concurrent.futures as cf

    import torch

    import synth
    from fp4_expert_ffn_amd import moe_blob_bytes
    from fp4_expert_ffn_amd.layer import CachedDecoder, blob_of

    cfg = synth.A3B
    E, k, H, I = cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    LAYERS, SLOTS, TOKENS, FMT = 48, 2048, args.stream_tokens, "nvfp4"
    warm_tokens = args.warmup if args.warmup is not None else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stride = (moe_blob_bytes(FMT, H, I) + 255) // 256 * 256
    log(f"[bench] stream: pinned bank of {LAYERS * E} experts ({LAYERS * E * stride / 1e9:.2f} GB)")
    t0 = time.perf_counter()
    # pinned chunks of 96 blobs (torch rounds each pinned allocation up to a power of two: 96 blobs fill 256 MiB)
    per_chunk = 96
    nkeys = LAYERS * E
    chunks = [torch.empty(min(per_chunk, nkeys - c0) * stride, dtype=torch.uint8, pin_memory=True)
              for c0 in range(0, nkeys, per_chunk)]
    chunks_np = [c.numpy() for c in chunks]

    def blob_view(key):
        c, i = divmod(key, per_chunk)
        return chunks[c][i * stride:(i + 1) * stride]

    def gen(key):
        l, e = divmod(key, E)
        b = blob_of(synth.expert(FMT, H, I, config=4, layer=l, expert_id=e))
        c, i = divmod(key, per_chunk)
        chunks_np[c][i * stride:i * stride + b.size] = b
        return key

    workers = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for i, _ in enumerate(ex.map(gen, range(LAYERS * E))):
            if (i + 1) % 1024 == 0:
                log(f"[bench]   {i + 1} experts generated ({time.perf_counter() - t0:.0f} s)")
    log(f"[bench] bank ready in {time.perf_counter() - t0:.1f}s; routing and activations")
    logits = synth.stream_routing(TOKENS, LAYERS, E)
    xs = np.empty((TOKENS, LAYERS, H), np.uint16)
    for t in range(TOKENS):
        for l in range(LAYERS):
            xs[t, l] = synth.stream_activations(t, l, H)[0]
    lg_d = torch.from_numpy(logits).to(dev)
    x_d = torch.from_numpy(xs.view(np.int16)).to(dev)

    dec = CachedDecoder(num_layers=LAYERS, num_experts=E, k=k, H=H, I=I, fmt=FMT, num_slots=SLOTS,
                        host_blob=lambda l, e: blob_view(l * E + e), device=dev)
    sh = torch.cuda.current_stream().cuda_stream

    # measured pinned host -> device rate: 128 slots in one copy on the copy stream
    n_cp = per_chunk
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(dec.copy_stream):
        dec.pool[:n_cp * stride].copy_(chunks[0], non_blocking=True)
        torch.cuda.synchronize()
        ev0.record()
        dec.pool[:n_cp * stride].copy_(chunks[1], non_blocking=True)
        ev1.record()
    torch.cuda.synchronize()
    h2d_peak = n_cp * stride / (ev0.elapsed_time(ev1) * 1e-3) / 1e9

    def run(t0_, t1_):
        for t in range(t0_, t1_):
            for l in range(LAYERS):
                dec.step_fast(l, x_d[t, l:l + 1], lg_d[t, l:l + 1], sh)

    log(f"[bench] warmup {warm_tokens} tokens, then {TOKENS} tokens from a cold cache")
    run(0, warm_tokens)
    torch.cuda.synchronize()
    dec.reset()
    t_start = time.perf_counter()
    n64 = min(64, TOKENS)
    run(0, n64)
    torch.cuda.synchronize()
    h64, m64, _ = dec.stats()
    log(f"[bench]   {n64} tokens in {time.perf_counter() - t_start:.2f} s")
    run(n64, TOKENS)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    hits, misses, nbytes = dec.stats()
    value = TOKENS / wall

    # a resize to half the slots between steps: the kept (most recent) blobs
    # are copied device to device, one slot read and written each
    from fp4_expert_ffn_amd import moe_cache_resize
    half = SLOTS // 2
    kept = min(half, SLOTS, misses)
    new_pool = torch.empty(half * stride, dtype=torch.uint8, device="cuda")
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record()
    moe_cache_resize(dec.cache, half, new_pool)
    r1.record()
    torch.cuda.synchronize()
    dec.pool = new_pool
    rs_ms = r0.elapsed_time(r1)
    rs_gbs = 2 * kept * stride / (rs_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] timing the CPU oracle on a bounded sample")

        def run_one(n):
            t, l = divmod(n, LAYERS)
            ids, w = oracle.moe.route(logits[t, l:l + 1], k)
            wts = {}

            def weights(e):
                if e not in wts:
                    wts[e] = oracle.moe.dequant_expert(synth.expert(FMT, H, I, config=4, layer=l, expert_id=e))
                return wts[e]
            oracle.moe.token_output(0, xs[t, l:l + 1], ids[0], w[0], weights)
        val, n, thr, dt = oracle_baseline(run_one, 1, args.cpu_budget)
        cpu = {"value": round(val / LAYERS, 4), "unit": "tokens/s", "cores": thr, "kind": "oracle",
               "sample": f"{n} (token, layer) steps of the stream, each generating and dequantising its 8 experts "
                         f"({dt:.1f} s); tokens/s = steps/s / {LAYERS} layers"}

    hit_rate = hits / max(hits + misses, 1)
    hit_late = (hits - h64) / max(hits - h64 + misses - m64, 1)
    h2d = nbytes / wall / 1e9
    line = {
        "metric": "MoE-stack decode tokens/s (48 layers through the expert cache)",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": TOKENS,
        "warmup": warm_tokens,
        "ms_per_step": round(wall / TOKENS * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4xbf16->f32",
        "data": "synthetic (seeded; weights N(0,0.02) quantised, activations N(0,1) bf16 per (token, layer), "
                "Zipf(1.1) routing with 0.6 repeat of the previous token's experts)",
        "config": {"workload": "cached decode stream: 48 A3B-like NVFP4 layers (hidden 2048, 128 experts, top-8, "
                               f"inter 768) in pinned host memory, 2048 HBM slots, {TOKENS} tokens at batch 1, "
                               "cold start",
                   "layers": LAYERS, "slots": SLOTS, "tokens": TOKENS, "parallelism": "single GPU"},
        "roofline": {"bound": "h2d", "achieved": round(h2d, 2), "peak": round(h2d_peak, 2), "unit": "GB/s",
                     "frac": round(h2d / h2d_peak, 4), "traffic": None,
                     "kernel": "hipMemcpyAsync pinned host -> HBM slot (miss fills)",
                     "peak_source": f"measured: one {n_cp}-slot pinned copy on the copy stream"},
        "cache": {"hits": hits, "misses": misses, "hit_rate": round(hit_rate, 4),
                  "hit_rate_tokens_64_511": round(hit_late, 4), "misses_per_token": round(misses / TOKENS, 2),
                  "bytes_filled": nbytes},
        "resize": {"slots": f"{SLOTS}->{half}", "kept_blobs": kept, "ms": round(rs_ms, 3),
                   "hbm_GBps": round(rs_gbs, 1), "hbm_frac": round(rs_gbs / 8000.0, 4),
                   "bytes_per_blob": 2 * stride, "kind": "device-to-device copies of the kept blobs"},
        "cpu_baseline": cpu,
    }
    dec.close()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
