#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE decode layer on one MI355X.

A step is one whole layer -- one moe_layer call (router GEMV + top-k, the sort
by expert, every active expert's fused dequant GEMVs and the weighted combine
plus the shared expert; --three-calls times moe_route, moe_sort_by_expert and
moe_mxfp4_forward instead) -- on the next of `--sets` distinct layer weight
sets, so consecutive steps never reuse expert weights and the 256 MB Infinity
Cache cannot serve them.  The K timed steps are replayed from HIP graphs
(every graph is replayed once before timing); the timed pass runs five times
and the median is reported.  Inputs are resident in HBM before the timed
region starts.

The default run (ling_m1) prints one JSON line for M = 1 with the M = 4
verify workload (ling_m4_mtp) nested under "ling_m4_mtp":
  value         layer GB/s: algorithmic bytes of a layer / time per layer
  ms_per_step   time per layer
  expert_rate   the experts' MXFP4 bytes / (gate/up + down kernel time), the
                kernels timed with HIP events bound to their own begin/end
  roofline      the dominant kernel (gate/up: two thirds of the expert bytes):
                its weight bytes per launch / mean launch duration
  cpu_baseline  the float64 oracle on a bounded sample of the same workload
                (all host threads, and one thread)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer µs & HBM GB/s (% of 8 TB/s), 2560×768×512e top-8, M=1/4"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes_per_expert(H, I):
    return 2 * I * (H // 2 + H // 32) + H * (I // 2 + I // 32)


def gateup_bytes_per_expert(H, I):
    return 2 * I * (H // 2 + H // 32)


def layer_bytes(wl, D):
    """Algorithmic bytes of one layer: every weight the method must read once
    (router, D active routed experts + shared), activations in, output out."""
    bias = 0
    if wl.routing == "overlap":
        bias = wl.M * wl.E * 4
    elif wl.routing == "zipf":
        bias = wl.E * 4
    expert = (D + int(wl.shared)) * expert_bytes_per_expert(wl.H, wl.I)
    return expert, wl.E * wl.H * 4 + wl.M * wl.H * 2 + wl.M * wl.H * 4 + bias + expert


class Prefetcher:
    """Expert prefetch beside the layers: on a side stream forked from the
    current one, moe_prefetch_select ranks a synthetic draft pass's routing of
    each layer set of a window, and moe_prefetch_experts reads the listed
    experts (gate/up and down); join() makes the current stream wait for it.  The
    draft keeps each of the set's true routed experts with probability
    `accuracy` (synth.draft_ids); the list holds the shared expert and every
    drafted expert."""

    def __init__(self, torch, binding, synth, wl, sets, weights, true_ids, accuracy, window, parts=3):
        import numpy as np
        self.torch, self.B, self.wl, self.weights = torch, binding, wl, weights
        self.accuracy, self.window, self.parts = accuracy, window, parts
        rng = np.random.default_rng(1000 + wl.seed)
        drafts = [synth.draft_ids(t, wl.E, accuracy, rng) for t in true_ids]
        self.hits = sum(len(set(d.ravel()) & set(t.ravel())) for d, t in zip(drafts, true_ids))
        self.needed = sum(len(set(t.ravel())) for t in true_ids)
        self.n_ids = wl.M * wl.k
        self.max_n = self.n_ids + int(wl.shared)
        self.drafts = [torch.tensor(d.reshape(-1), dtype=torch.int32, device="cuda") for d in drafts]
        self.lst = torch.zeros(self.max_n, dtype=torch.int32, device="cuda")
        self.num = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.cs = torch.zeros(self.max_n, dtype=torch.int32, device="cuda")
        self.side = torch.cuda.Stream()
        self.done = torch.cuda.Event()

    def fork(self, set_ids):
        """Prefetch the listed layer sets, in order, on the side stream."""
        t = self.torch
        self.side.wait_stream(t.cuda.current_stream())
        s = self.side.cuda_stream
        for set_idx in set_ids:
            self.B.moe_prefetch_select(self.drafts[set_idx], self.n_ids, self.wl.E, int(self.wl.shared),
                                       self.max_n, self.lst, self.num, s)
            self.B.moe_prefetch_experts(self.weights[set_idx], self.lst, self.num, self.max_n, self.parts,
                                        self.cs, s)
        self.done.record(self.side)

    def join(self):
        self.torch.cuda.current_stream().wait_event(self.done)

    def describe(self):
        return {"accuracy": self.accuracy, "window": self.window,
                "parts": {1: "gate/up", 2: "down", 3: "gate/up + down"}[self.parts],
                "list": "shared + drafted experts by heat",
                "predicted_fraction_of_needed_experts": round(self.hits / max(self.needed, 1), 4),
                "when": "the W layers after the next W, read on a side stream while those run"}


def device_sets(torch, wl, nsets):
    """x / router / bias from the seeded numpy generator; the expert banks are
    filled on the device with torch's seeded generator (same distribution:
    uniform code bytes, scale bytes uniform over [120, 127]) -- 1.6 GB per set
    would take about a minute per 40 sets on the host."""
    from mxfp4_expert_weight_amd import synth
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, to_device
    out = []
    n, H, I = wl.E + 1, wl.H, wl.I
    for l in range(nsets):
        ls = synth.layer_set(wl, l, banks=False)
        g = torch.Generator(device="cuda")
        g.manual_seed(wl.seed * 1_000_003 + l)
        u8 = dict(dtype=torch.uint8, device="cuda", generator=g)
        out.append(DeviceLayerSet(
            to_device(ls.x_bits), to_device(ls.w_router), to_device(ls.bias), ls.bias_row_stride,
            torch.randint(0, 256, (n, 2 * I, H // 2), **u8), torch.randint(120, 128, (n, 2 * I, H // 32), **u8),
            torch.randint(0, 256, (n, H, I // 2), **u8), torch.randint(120, 128, (n, H, I // 32), **u8),
            wl.M, H, I, wl.E, wl.k, wl.shared))
    torch.cuda.synchronize()
    return out


# the translation unit that defines each profiled kernel
KERNEL_SOURCE = {"gateup_kernel": "forward.hip", "decode_gateup_kernel": "decode.hip",
                 "decode_down_kernel": "decode.hip", "lmhead_fp8_kernel": "lmhead.hip",
                 "lmhead_mfma_kernel": "lmhead.hip"}


def gateup_kernel_name(wl, three_calls=False, hinted=False):
    """The kernel that streams the gate/up weights on this workload: moe_layer
    takes the decode path (one routing-and-gate/up kernel, then one down
    kernel) for up to 4 tokens at H = 2560, I = 768 without a hint list."""
    if wl.M <= 4 and (wl.H, wl.I) == (2560, 768) and not three_calls and not hinted:
        return "decode_gateup_kernel"
    return "gateup_kernel"


def kernel_source_hash(kernel=None):
    """sha256 over the kernel's translation unit and every local header it
    includes (all HIP sources and the header when no kernel is named): a
    traffic figure measured on other sources is stale."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "mxfp4_expert_weight_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    if kernel is None:
        files = [os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h"))]
        files.append(os.path.join(inc, "moe_mxfp4.h"))
    else:
        files, todo = [], [os.path.join(csrc, KERNEL_SOURCE[kernel])]
        while todo:
            f = todo.pop()
            if f in files:
                continue
            files.append(f)
            for name in re.findall(r'^#include "([^"]+)"', open(f).read(), re.M):
                for d in (csrc, inc):
                    if os.path.exists(os.path.join(d, name)):
                        todo.append(os.path.join(d, name))
                        break
    h = hashlib.sha256()
    for f in sorted(files, key=os.path.basename):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(workload, kernel="gateup_kernel"):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_summary(dirs, kernel):
    """Summarise rocprofv3 csv output directories (kernel stats and per-dispatch
    counters) as text."""
    import csv
    import glob
    import statistics
    lines = []
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
            lines.append(f"kernel stats ({os.path.relpath(f, d)}):")
            lines.append(f"  {'kernel':64s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'%':>6s}")
            for r in csv.DictReader(open(f)):
                lines.append(f"  {r['Name'][:64]:64s} {r['Calls']:>7s} {float(r['AverageNs']) / 1e3:9.2f} "
                             f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                             f"{float(r['Percentage']):6.1f}")
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            per = {}
            for r in csv.DictReader(open(f)):
                key = (r["Kernel_Name"], r["Counter_Name"])
                per.setdefault(key, []).append(float(r["Counter_Value"]))
            lines.append(f"counters per dispatch ({os.path.relpath(f, d)}):")
            for (kn, cn), vals in sorted(per.items()):
                if kernel and kernel not in kn and "elementwise" not in kn and "copy" not in kn.lower():
                    continue
                lines.append(f"  {kn[:64]:64s} {cn:12s} n={len(vals):6d} mean={statistics.mean(vals):14.1f} "
                             f"median={statistics.median(vals):14.1f}")
    print("\n".join(lines))


def blas_threads():
    """Threads of the BLAS the oracle's matrix products run on."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_layers(wl, seconds_budget, w4a8):
    """Time the oracle as it stands on host-generated sets of the workload,
    set after set, until the budget is spent: whole layers for M <= 8, else 4
    sampled tokens per set with the time scaled to the M tokens."""
    import numpy as np

    import oracle
    from mxfp4_expert_weight_amd import synth
    times, nbytes = [], []
    start = time.time()
    l = 0
    while l < wl.sets and (time.time() - start) < seconds_budget:
        ls = synth.layer_set(wl, l)
        t0 = time.perf_counter()
        if wl.M <= 8:
            layer = oracle.moe_layer_w4a8 if w4a8 else oracle.moe_layer
            r = layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k, wl.shared)
            D = r["num_active"]
            frac = 1.0
        else:   # large batches: a bounded token sample, scaled to the layer
            sample = list(range(0, wl.M, max(1, wl.M // 4)))[:4]
            tokens_fn = oracle.moe_layer_w4a8_tokens if w4a8 else oracle.moe_layer_tokens
            tokens_fn(sample, ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k,
                      wl.shared)
            D = int(np.unique(oracle.topk_softmax(oracle.router_logits(
                oracle.bf16_bits_to_f64(ls.x_bits), ls.w_router, ls.bias), wl.k)[0]).size)
            frac = len(sample) / wl.M
        times.append((time.perf_counter() - t0) / frac)
        nbytes.append(layer_bytes(wl, D)[1])
        l += 1
    sec = sum(times) / len(times)
    return sec, sum(nbytes) / len(nbytes) / sec / 1e9, len(times)


def cpu_baseline(wl, seconds_budget=10.0, w4a8=False, one_thread=True):
    """The oracle as it stands, on host-generated sets of the same workload:
    once with the BLAS's own thread count, once on one thread."""
    threads = blas_threads()
    sec, gbs, n = _oracle_layers(wl, seconds_budget, w4a8)
    kind = "whole layers" if wl.M <= 8 else "4 tokens per layer, time scaled to M tokens"
    out = {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} layer sets of {wl.name} ({kind}); {sec * 1e3:.1f} ms per layer",
           "us_per_layer": sec * 1e6, "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    if one_thread:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                sec1, gbs1, n1 = _oracle_layers(wl, seconds_budget, w4a8)
            out["one_thread"] = {"value": gbs1, "unit": "GB/s", "cores": 1, "us_per_layer": sec1 * 1e6,
                                 "sample": f"{n1} layer sets of {wl.name} ({kind})"}
        except ImportError:
            out["one_thread"] = None
    return out


def bench_lmhead(torch, binding, synth, args):
    """The FP8 LM head (157,184 x 2,560, E4M3 codes + fp32 row scales) for M
    tokens: K projections replayed from a HIP graph over enough distinct code
    sets that the 256 MB Infinity Cache cannot hold them; value = bytes the
    projection must read (codes, scales, x) and write (logits) per second."""
    M = 4 if args.workload == "lmhead_fp8_m4" else 1
    V, H = synth.LMHEAD_VOCAB, synth.LMHEAD_HIDDEN
    nsets = args.sets or 4
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    sets = []
    for _ in range(nsets):
        codes = torch.randint(0, 256, (V, H), dtype=torch.uint8, device="cuda", generator=g)
        codes = torch.where((codes & 0x7F) == 0x7F, codes ^ 1, codes)       # no NaN codes
        scales = torch.exp2(torch.rand(V, device="cuda", generator=g) - 13.0)
        sets.append((codes, scales))
    x = torch.from_numpy(synth.lmhead_set(M, 1, H, seed=5).x_bits.view("int16")).cuda()
    out = torch.empty((M, V), dtype=torch.float32, device="cuda")
    for c, sc in sets:
        binding.moe_lmhead_fp8_logits(x, c, sc, M, V, H, out)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for c, sc in sets:
            binding.moe_lmhead_fp8_logits(x, c, sc, M, V, H, out)
    torch.cuda.current_stream().wait_stream(st)
    with torch.cuda.graph(gr):
        for c, sc in sets:
            binding.moe_lmhead_fp8_logits(x, c, sc, M, V, H, out)
    steps = max(nsets, args.steps // nsets * nsets)
    for _ in range(max(1, args.warmup // nsets)):
        gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps // nsets):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = V * H + V * 4 + M * H * 2 + M * V * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the projection kernel: the matrix cores take 2+ tokens on rows a multiple of 256
    lm_kernel = "lmhead_mfma_kernel" if M >= 2 and H % 256 == 0 else "lmhead_fp8_kernel"
    log(f"[bench] lmhead M={M}: {steps} projections, {ms * 1e3:.2f} us each, {nbytes / 1e6:.1f} MB, "
        f"{gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")
    out_json = {
        "metric": "FP8 LM-head projection GB/s (157184x2560 E4M3, fp32 row scales)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "vocab": V, "hidden": H, "weights": "E4M3 + fp32/row",
                   "activations": "bf16", "code_sets_rotated": nsets},
        "us_per_projection": ms * 1e3,
        "roofline": {"bound": "hbm", "kernel": lm_kernel, "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(args.workload, lm_kernel)},
    }
    if not args.no_cpu_baseline:
        out_json["cpu_baseline"] = lmhead_cpu_baseline(synth, M, V, H)
    print(json.dumps(out_json), flush=True)


def lmhead_cpu_baseline(synth, M, V, H, seconds_budget=10.0):
    """The oracle's float64 projection of M tokens onto samples of 8,192 head
    rows, repeated within the budget; GB/s of the sampled rows' bytes."""
    import statistics

    import oracle
    rows = 8192
    s = synth.lmhead_set(M, rows, H, seed=11)
    nbytes = rows * H + rows * 4 + M * H * 2 + M * rows * 4
    times = []
    t_end = time.perf_counter() + seconds_budget
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        oracle.lmhead_logits(s.x_bits, s.codes, s.scales)
        times.append(time.perf_counter() - t0)
    sec = statistics.median(times)
    return {"value": nbytes / sec / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{len(times)} projections of {M} token(s) onto {rows} of the {V} rows (H = {H}); "
                      f"{sec * 1e3:.1f} ms each, {sec * V / rows * 1e3:.0f} ms scaled to the whole head"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="ling_m1",
                    help="a MoE workload (ling_m1, ling_m4_mtp, ling_m32_zipf, ling_m512_prefill, tiny) "
                         "or the FP8 LM head (lmhead_fp8, lmhead_fp8_m4)")
    ap.add_argument("--sets", type=int, default=None, help="layer sets rotated (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--w4a8", action="store_true",
                    help="the W4A8 variant (moe_layer_w4a8: MXFP8 activations into the experts)")
    ap.add_argument("--prefetch", type=float, default=None, metavar="ACC",
                    help="prefetch each next layer's predicted experts (moe_prefetch_select + "
                         "moe_prefetch_experts on a side stream) while the current layer runs; the "
                         "synthetic draft keeps each true expert with probability ACC")
    ap.add_argument("--prefetch-window", type=int, default=4, metavar="W",
                    help="with --prefetch: layers prefetched per fork of the side stream; the layers "
                         "W..2W-1 ahead are read while the next W run")
    ap.add_argument("--hint", type=float, default=None, metavar="ACC",
                    help="moe_layer_hinted: each layer gets the experts a synthetic draft predicts (each true "
                         "expert kept with probability ACC), sorted by moe_sort_by_expert before timing")
    ap.add_argument("--gap-kernels", type=int, default=0, metavar="N",
                    help="before each layer, N small elementwise kernels on a 256 KB tensor that stays in "
                         "L2: a stand-in for the non-MoE work between two layers that leaves HBM idle "
                         "(with --prefetch, each layer's own experts are prefetched during it)")
    ap.add_argument("--phases", action="store_true",
                    help="the decode path's per-workgroup phase timestamps (moe_layer_probe) instead of the bench")
    ap.add_argument("--single", action="store_true",
                    help="ling_m1 alone (the default run also measures ling_m4_mtp into the same line)")
    ap.add_argument("--three-calls", action="store_true",
                    help="time moe_route + moe_sort_by_expert + moe_mxfp4_forward instead of moe_layer")
    ap.add_argument("--no-helpers", action="store_true",
                    help="batches: every expert kernel on the one stream (no helper streams)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (reference for rocprof byte counters)")
    ap.add_argument("--profile-summary", nargs="+", metavar="DIR",
                    help="print a text summary of rocprofv3 csv output directories and exit")
    ap.add_argument("--kernel", default="gateup_kernel", help="kernel kept in --profile-summary counters")
    ap.add_argument("--source-hash", nargs="?", const="", default=None, metavar="KERNEL",
                    help="print the sha256 of KERNEL's sources (of all kernel sources without KERNEL) and exit")
    args = ap.parse_args()
    if args.profile_summary:
        profile_summary(args.profile_summary, args.kernel)
        return
    if args.source_hash is not None:
        print(kernel_source_hash(args.source_hash or None))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from mxfp4_expert_weight_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 3 x 1 GiB device-to-device copies")
        return

    if args.workload.startswith("lmhead"):
        bench_lmhead(torch, binding, synth, args)
        return

    wl = synth.WORKLOADS[args.workload]
    if args.phases:
        phase_table(torch, binding, synth, args, wl)
        return
    out = bench_moe(torch, binding, synth, args, wl, cpu=not args.no_cpu_baseline)
    if args.workload == "ling_m1" and not args.single and not (args.hint is not None or args.prefetch is not None
                                                              or args.gap_kernels or args.three_calls):
        # the M = 4 verify workload of the same metric, nested in the same line
        torch.cuda.empty_cache()
        m4 = bench_moe(torch, binding, synth, args, synth.WORKLOADS["ling_m4_mtp"], cpu=not args.no_cpu_baseline,
                       cpu_budget=5.0, one_thread=False)
        keep = ("us_per_layer", "value", "unit", "ms_per_step", "layer_frac_of_hbm_peak", "expert_bytes_per_layer",
                "expert_rate", "read_floor", "roofline", "mean_distinct_experts", "config", "timed_passes_us_per_layer",
                "cpu_baseline")
        out["ling_m4_mtp"] = {k: m4[k] for k in keep if k in m4}
        out["t_m4_over_t_m1"] = m4["us_per_layer"] / out["us_per_layer"]
    print(json.dumps(out), flush=True)


def read_floor(torch, binding, wl, sets, true_ids, hev, order):
    """The read-bandwidth floor of each set's bytes (moe_read_probe: one
    kernel that only reads, every load of a workgroup in flight at once),
    launched eagerly over the sets in `order`, mean kernel time per launch:
    the gate/up weights of the layer's experts (routed + shared), their down
    weights, all of their weights in one kernel, and the router's weights."""
    import numpy as np
    H, I, E = wl.H, wl.I, wl.E
    gq, gs = 2 * I * (H // 2), 2 * I * (H // 32)             # bytes per expert
    dq, ds = H * (I // 2), H * (I // 32)
    def ranges(d, ids, parts):
        experts = sorted(set(int(e) for e in np.asarray(ids).ravel())) + ([E] if wl.shared else [])
        out = []
        for e in experts:
            if "gateup" in parts:
                out += [(d.w13_q.data_ptr() + e * gq, gq), (d.w13_s.data_ptr() + e * gs, gs)]
            if "down" in parts:
                out += [(d.w2_q.data_ptr() + e * dq, dq), (d.w2_s.data_ptr() + e * ds, ds)]
        return out
    kinds = {"gateup": ("gateup",), "down": ("down",), "experts": ("gateup", "down"), "router": ()}
    prepared = {k: [] for k in kinds}
    for d, ids in zip(sets, true_ids):
        for k, parts in kinds.items():
            r = [(d.w_router.data_ptr(), E * H * 4)] if k == "router" else ranges(d, ids, parts)
            mb = max(sz for _, sz in r)
            a = torch.tensor([x for x, _ in r], dtype=torch.int64, device="cuda")
            z = torch.tensor([sz for _, sz in r], dtype=torch.int64, device="cuda")
            words = binding.read_probe_words(len(r), mb)
            prepared[k].append((a, z, len(r), mb, torch.empty((words,), dtype=torch.int32, device="cuda"), words,
                                sum(sz for _, sz in r)))
    res = {}
    for k in kinds:
        evs = [(hev.create(), hev.create()) for _ in order]
        for (i, (e0, e1)) in zip(order, evs):
            a, z, n, mb, out, words, _ = prepared[k][i]
            binding.moe_read_probe(a, z, n, mb, out, words, e0, e1)
        torch.cuda.synchronize()
        us = sum(hev.elapsed_ms(e0, e1) for e0, e1 in evs) / len(evs) * 1e3
        nbytes = sum(prepared[k][i][6] for i in order) / len(order)
        for e0, e1 in evs:
            hev.destroy(e0)
            hev.destroy(e1)
        res[k] = {"us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9}
    log("[floor] " + ", ".join(f"{k} {v['us']:.2f} us ({v['bytes'] / 1e6:.1f} MB, {v['gbs']:.0f} GB/s)"
                               for k, v in res.items()))
    return res


def phase_table(torch, binding, synth, args, wl):
    """Where a decode layer's time goes: moe_layer_probe's per-workgroup
    timestamps (100 MHz) over --steps layers run back to back on the rotating
    sets, each workgroup's phases in microseconds from its gate/up kernel's
    first workgroup start.  Prints one JSON line."""
    import statistics

    from mxfp4_expert_weight_amd.layer import LayerBuffers
    nsets = args.sets or wl.sets
    sets = device_sets(torch, wl, nsets)
    buf = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    n = binding.moe_layer_probe_stamps(wl.M, wl.k, wl.E, wl.H, wl.I)
    assert n > 0, "the decode path does not cover this workload"
    steps = max(args.steps, 1)
    stamps = torch.zeros((steps, n), dtype=torch.int64, device="cuda")
    for i in range(steps):
        d = sets[i % nsets]
        binding.moe_layer_probe(d.x, d.w_router, d.bias, d.bias_row_stride, d.weights(), d.M, d.k, buf.logits,
                                buf.ids, buf.weights, buf.offsets, buf.pairs, buf.active, buf.num_active, buf.y,
                                buf.ws, buf.ws_bytes, stamps[i], n)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().reshape(steps, -1, 16).astype("float64") / 100.0   # 100 MHz ticks -> us
    names = ["gate/up start", "logits loaded", "top-k threshold", "top-k done", "routing barrier",
             "slot known", "weights issued", "first weights used", "h written",
             "down start", "record loaded", "down loads issued", "down first weights", "down done",
             "unused 14", "unused 15"]
    rows = {k: [] for k in names}
    ends = {"gate/up last start": [], "gate/up end": [], "down first start": [], "down end": []}
    for s_ in st:
        t0 = s_[:, 0][s_[:, 0] > 0].min()
        for j, k in enumerate(names):
            v = s_[:, j][s_[:, j] > 0] - t0
            rows[k].append((statistics.median(v), float(v.max())) if len(v) else (None, None))
        gs = s_[:, 0][s_[:, 0] > 0] - t0
        ends["gate/up last start"].append(float(gs.max()))
        ends["gate/up end"].append(float((s_[:, 8][s_[:, 8] > 0] - t0).max()))
        ends["down first start"].append(float((s_[:, 9][s_[:, 9] > 0] - t0).min()))
        ends["down end"].append(float((s_[:, 13][s_[:, 13] > 0] - t0).max()))
    table = {k: {"median_us": statistics.median([m for m, _ in v if m is not None]),
                 "max_us": statistics.median([x for _, x in v if x is not None])}
             for k, v in rows.items() if any(m is not None for m, _ in v)}
    for k, v in ends.items():
        table[k] = {"median_us": statistics.median(v)}
    for k, v in table.items():
        log(f"[phases] {wl.name} {k:20s} " + " ".join(f"{a}={b:.2f}" for a, b in v.items()))
    print(json.dumps({"workload": wl.name, "layers": steps, "phases_from_gateup_start_us": table,
                      "what": "median over layers of the median (max) over workgroups"}), flush=True)


def bench_moe(torch, binding, synth, args, wl, cpu=True, cpu_budget=10.0, one_thread=True):
    """Measure one MoE workload; returns the bench line's fields."""
    import statistics

    from mxfp4_expert_weight_amd.layer import HelperStreams, HipEvents, LayerBuffers, run_layer
    nsets = args.sets or wl.sets
    t0 = time.time()
    sets = device_sets(torch, wl, nsets)
    log(f"[bench] {nsets} layer sets of {wl.name} on the device in {time.time() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    buf = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    weights = [d.weights() for d in sets]
    # batches run their matrix-core experts on two helper streams of ours
    helpers = HelperStreams() if wl.M > 4 and not args.no_helpers else None

    # one eager pass: loads the kernels and records each set's distinct-expert count
    D, G, true_ids = [], [], []
    for d, w in zip(sets, weights):
        run_layer(d, buf, w, w4a8=args.w4a8, helpers=helpers)
        D.append(int(buf.num_active.item()))
        G.append(buf.header()["gemv_experts"])   # experts on the GEMV path (the timed kernels)
        true_ids.append(buf.ids.cpu().numpy())
    log(f"[bench] distinct routed experts per set: min {min(D)} max {max(D)} mean {sum(D) / len(D):.2f}")

    hints = None
    if args.hint is not None:             # the draft's predicted experts of every set, ascending, on the device
        import numpy as np
        rng = np.random.default_rng(2000 + wl.seed)
        hints = []
        offs = torch.empty(wl.E + 1, dtype=torch.int32, device="cuda")
        prs = torch.empty(wl.M * wl.k, dtype=torch.int32, device="cuda")
        hit = need = 0
        for t in true_ids:
            dr = synth.draft_ids(t, wl.E, args.hint, rng)
            hit += len(set(dr.ravel()) & set(t.ravel()))
            need += len(set(t.ravel()))
            act = torch.full((wl.E,), -1, dtype=torch.int32, device="cuda")
            num = torch.zeros(1, dtype=torch.int32, device="cuda")
            binding.moe_sort_by_expert(torch.tensor(dr.reshape(-1), dtype=torch.int32, device="cuda"), wl.M, wl.k,
                                       wl.E, offs, prs, act, num)
            hints.append((act, num))
        torch.cuda.synchronize()
        hint_frac = hit / max(need, 1)

    def run_step(i, gu_ev=None, dn_ev=None):
        l = i % nsets
        if hints is not None:
            d = sets[l]
            binding.moe_layer_hinted(d.x, d.w_router, d.bias, d.bias_row_stride, weights[l], d.M, d.k, buf.logits,
                                     buf.ids, buf.weights, buf.offsets, buf.pairs, buf.active, buf.num_active, buf.y,
                                     buf.ws, buf.ws_bytes, hints[l][0], hints[l][1],
                                     *(gu_ev if gu_ev is not None else (None, None)))
        else:
            run_layer(sets[l], buf, weights[l], fused=not args.three_calls, w4a8=args.w4a8, helpers=helpers,
                      gateup_events=gu_ev, down_events=dn_ev)

    pf = None
    if args.prefetch is not None:
        assert args.prefetch_window >= 1 and nsets % args.prefetch_window == 0, \
            "the prefetch window must divide the number of layer sets"
        pf = Prefetcher(torch, binding, synth, wl, sets, weights, true_ids, args.prefetch, args.prefetch_window)

    gap = torch.zeros(1 << 16, device="cuda") if args.gap_kernels else None

    def run_gap():
        for _ in range(args.gap_kernels):
            gap.add_(1.0)

    def capture(first, n, prefetch, layers=True):
        """A graph of steps first .. first+n-1 (layer set = step mod nsets)."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()

        def steps():
            W = args.prefetch_window
            for i in range(first, first + n):
                if gap is not None:
                    # the stand-in gap; with the prefetch, this layer's experts are read during it
                    if prefetch:
                        pf.fork([i % nsets])
                    run_gap()
                    if prefetch:
                        pf.join()
                    if layers:
                        run_step(i)
                    continue
                if prefetch and (i - first) % W == 0:
                    if i != first:
                        pf.join()
                    pf.fork([(i + W + j) % nsets for j in range(W)])
                run_step(i)
            if prefetch and gap is None:
                pf.join()

        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            steps()
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(g):
            steps()
        return g

    def timed_replays(prefetch, layers=True, passes=5):
        """K = args.steps steps: a graph per pass over the sets plus one for the
        remainder, each replayed once before timing (and --warmup steps of
        replays in all); then `passes` timed passes of exactly K steps, each
        bracketed by synchronisations.  Returns the per-pass times (ms)."""
        K = args.steps
        reps, rem = K // nsets, K % nsets
        g_full = capture(0, nsets, prefetch, layers) if reps else None
        g_rem = capture(reps * nsets, rem, prefetch, layers) if rem else None

        def one_pass():
            for _ in range(reps):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()

        one_pass()                                   # every graph replayed once before timing
        for _ in range(math.ceil(max(args.warmup - K, 0) / max(K, 1))):
            one_pass()
        torch.cuda.synchronize()
        ms = []
        for _ in range(passes):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record()
            one_pass()
            ev1.record()
            torch.cuda.synchronize()
            ms.append(ev0.elapsed_time(ev1))
        return ms

    plain_ms = gap_ms = None
    if gap is not None:
        gap_ms = statistics.median(timed_replays(False, layers=False))
        log(f"[bench] the gap alone ({args.gap_kernels} kernels): {gap_ms / args.steps * 1e3:.2f} us per step")
    if pf is not None:
        plain_ms = statistics.median(timed_replays(False))
        log(f"[bench] without prefetch: {plain_ms / args.steps * 1e3:.2f} us per step")
    passes = timed_replays(pf is not None)
    ms_total = statistics.median(passes)
    if gap is not None:                  # the layer's share of each step
        log(f"[bench] gap + layer: {ms_total / args.steps * 1e3:.2f} us per step")
        ms_total -= gap_ms
        passes = [p - gap_ms for p in passes]
        if plain_ms is not None:
            plain_ms -= gap_ms
    ms_per_step = ms_total / args.steps
    step_sets = [i % nsets for i in range(args.steps)]
    exp_b = [layer_bytes(wl, D[l])[0] for l in step_sets]
    lay_b = [layer_bytes(wl, D[l])[1] for l in step_sets]
    layer_gbs = sum(lay_b) / (ms_total * 1e-3) / 1e9
    log(f"[bench] {wl.name}: {args.steps} steps, median of {len(passes)} passes {ms_total:.3f} ms "
        f"({', '.join(f'{p / args.steps * 1e3:.2f}' for p in passes)} us/layer): "
        f"{ms_per_step * 1e3:.2f} us/layer, {layer_gbs:.0f} GB/s")

    # The GEMV gate/up and down kernels (for M <= 4 every expert runs on them;
    # gate/up is the dominant kernel, two thirds of the expert bytes): per-launch
    # durations from HIP events bound to each kernel's own begin/end timestamps,
    # over the same K steps run eagerly on the stream the kernels use.  Their
    # bytes are those of the experts the header reports on the GEMV path.
    hev = HipEvents()
    n_ev = min(args.steps, 2000)
    evs = [[hev.create() for _ in range(4)] for _ in range(n_ev)]
    torch.cuda.synchronize()
    W = args.prefetch_window
    if pf is not None and gap is None:   # the first window's experts, as the replays leave them
        pf.fork([step_sets[j % len(step_sets)] for j in range(W)])
    for i in range(n_ev):
        if gap is not None:
            if pf is not None:
                pf.fork([step_sets[i]])
            run_gap()
            if pf is not None:
                pf.join()
        elif pf is not None and i % W == 0:
            pf.join()
            pf.fork([(step_sets[i] + W + j) % nsets for j in range(W)])
        run_step(i, evs[i][:2], evs[i][2:])
    if pf is not None and gap is None:
        pf.join()
    torch.cuda.synchronize()
    gu_ms = sum(hev.elapsed_ms(e[0], e[1]) for e in evs) / n_ev
    dn_ms = None if hints is not None else sum(hev.elapsed_ms(e[2], e[3]) for e in evs) / n_ev
    for e in evs:
        for h in e:
            hev.destroy(h)
    gu_bytes = sum(G[step_sets[i]] * gateup_bytes_per_expert(wl.H, wl.I) for i in range(n_ev)) / n_ev
    gemv_exp_bytes = sum(G[step_sets[i]] * expert_bytes_per_expert(wl.H, wl.I) for i in range(n_ev)) / n_ev
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    log(f"[bench] gate/up kernel: {gu_ms * 1e3:.2f} us per launch, {gu_bytes / 1e6:.2f} MB, "
        f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")
    expert_rate = None
    if dn_ms is not None:
        rate = gemv_exp_bytes / ((gu_ms + dn_ms) * 1e-3) / 1e9
        expert_rate = {"value": round(rate, 2), "unit": "GB/s", "frac_of_hbm_peak": rate / HBM_PEAK_GBS,
                       "gateup_us": gu_ms * 1e3, "down_us": dn_ms * 1e3, "bytes": gemv_exp_bytes,
                       "what": "(experts on the GEMV path) x 3,133,440 B / (gate/up + down kernel time)"}
        log(f"[bench] down kernel: {dn_ms * 1e3:.2f} us per launch; expert rate {rate:.0f} GB/s "
            f"({rate / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    gu_kernel = gateup_kernel_name(wl, args.three_calls, hints is not None)
    floor = read_floor(torch, binding, wl, sets, true_ids, hev, [step_sets[i] for i in range(n_ev)])
    out = {
        "metric": METRIC,
        "value": round(layer_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name,
                   "entry": "moe_layer_ex (W4A8)" if args.w4a8 else ("three calls" if args.three_calls else "moe_layer"),
                   "M": wl.M, "hidden": wl.H, "inter": wl.I, "experts": wl.E,
                   "top_k": wl.k, "shared_expert": wl.shared, "routing": wl.routing,
                   "layer_sets_rotated": nsets, "weights": "MXFP4 (E2M1 + E8M0/32)",
                   "activations": "MXFP8 (E4M3 + E8M0/32) into the experts" if args.w4a8 else "bf16",
                   "helper_streams": helpers is not None},
        "us_per_layer": ms_per_step * 1e3,
        "timed_passes_us_per_layer": [p / args.steps * 1e3 for p in passes],
        "layer_bytes": sum(lay_b) / len(lay_b),
        "layer_frac_of_hbm_peak": layer_gbs / HBM_PEAK_GBS,
        # the routed and shared experts' MXFP4 bytes over the whole layer time
        "expert_bytes_per_layer": sum(exp_b) / len(exp_b),
        "expert_gbs": sum(exp_b) / (ms_total * 1e-3) / 1e9,
        "expert_frac_of_hbm_peak": sum(exp_b) / (ms_total * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "expert_rate": expert_rate,
        # the same bytes read by a kernel that only reads (moe_read_probe):
        # what the chip allows for each part, and how far each part is from it
        "read_floor": {
            "what": "mean kernel time of moe_read_probe over the timed sets: the layer's expert gate/up weights, "
                    "their down weights, all of them in one kernel, and the router weights",
            "gateup_us": floor["gateup"]["us"], "down_us": floor["down"]["us"],
            "experts_us": floor["experts"]["us"], "router_us": floor["router"]["us"],
            "experts_gbs": floor["experts"]["gbs"],
            "layer_over_experts_floor": ms_per_step * 1e3 / floor["experts"]["us"],
            "gateup_kernel_over_floor": (gu_ms * 1e3 / floor["gateup"]["us"]) if gu_kernel.startswith("decode") else None,
            "down_kernel_over_floor": (dn_ms * 1e3 / floor["down"]["us"])
            if gu_kernel.startswith("decode") and dn_ms is not None else None,
        },
        "mean_distinct_experts": sum(D[l] for l in step_sets) / len(step_sets),
        "roofline": {"bound": "hbm", "kernel": gu_kernel,
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(wl.name + ("_w4a8" if args.w4a8 else ""), gu_kernel),
                     "us_per_launch": gu_ms * 1e3, "bytes_per_launch": gu_bytes},
    }
    if hints is not None:
        out["roofline"]["traffic"] = None     # counters were taken without hints (wrong hints fetch more)
        out["config"]["entry"] = "moe_layer_hinted"
        out["config"]["hint"] = {"accuracy": args.hint, "predicted_fraction_of_needed_experts": round(hint_frac, 4),
                                 "list": "the draft's routed experts, ascending (moe_sort_by_expert)"}
    if gap is not None:
        out["config"]["gap_kernels"] = args.gap_kernels
        out["us_gap_per_step"] = gap_ms / args.steps * 1e3
    if pf is not None:
        out["config"]["prefetch"] = pf.describe()
        if gap is not None:
            out["config"]["prefetch"]["window"] = 1
            out["config"]["prefetch"]["when"] = "during the gap before the layer, on a side stream"
        out["us_per_layer_without_prefetch"] = plain_ms / args.steps * 1e3
        out["roofline"]["traffic"] = None     # counters were taken without the prefetch beside the layer
    del sets, weights, buf, pf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = cpu_baseline(wl, seconds_budget=cpu_budget, w4a8=args.w4a8, one_thread=one_thread)
    return out


if __name__ == "__main__":
    main()
