"""Benchmark of the MI355X attention backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one whole backward chain (preprocess, main, GQA reduce, dQ convert or dq2k) over one
batch of synthetic inputs resident in HBM.  The default workload is causal GQA, B=1, Hq=32, Hkv=8,
S=4096, D=128 with fp32 atomic dQ.  Prints one JSON line: whole-chain TFLOP/s, the main kernel's
MFMA roofline (its duration measured with HIP events recorded by the library on the launch stream)
and the CPU oracle timed on a bounded sample of the same workload.

FLOPs per visible (query, key) pair and head: 2 * (3 * Dqk + 2 * Dv) (S recompute, dP, dV, dQ,
dK); for a plain causal mask the dense count is halved, with a window or padding the visible
pairs are counted.

Inputs: Q, K, V, dO drawn by the seeded generator; O and LSE come from a float32 forward computed
with torch on the GPU (input preparation only, outside the timed region).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_backward_sdpa_amd import synth  # noqa: E402

METRIC = "attention-backward TFLOP/s and % of bf16 MFMA peak, S=4096 D=128 causal"
# dQ routes as sdpa_bwd_dq_route() reports them, and the kernel that ends each chain
ROUTE_NAMES = {0: "fp32 atomic", 2: "deterministic: dS panels + dq2k",
               3: "deterministic: fp32 dQ partials + ordered reduction",
               4: "deterministic: ordered relay"}
ROUTE_STAGE = {0: "dq_convert", 2: "dq2k", 3: "dq_reduce", 4: "dq_reduce"}
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (AMD's 2.5 PFLOP/s)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "main_kernel_traffic.json")
KERNEL_SOURCES = ["bwd_main.h", "common.h", "masks.h", "nvfp4.h"]


def kernel_source_hash():
    """Hash of the main kernel's sources with comments and whitespace removed, so that the traffic
    record stays valid across edits that do not change the code."""
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_backward_sdpa_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def visible_pairs(w, lens):
    """Visible (query, key) pairs summed over the batch (the mask rule, counted row by row)."""
    total = 0
    for b in range(w.B):
        L = w.Sq if lens is None else int(lens[b])
        Lk = w.Skv if lens is None else int(lens[b])
        i = np.arange(L)
        hi = np.minimum(i, Lk - 1) if w.causal else np.full(L, Lk - 1)
        lo = np.maximum(i - w.window_left, 0) if w.window_left >= 0 else np.zeros(L, dtype=np.int64)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


def algorithmic_flops(w, lens):
    per_pair = 2 * (3 * w.Dqk + 2 * w.Dv)
    if w.window_left < 0 and lens is None:
        return per_pair * w.Sq * w.Skv * (0.5 if w.causal else 1.0) * w.B * w.Hq
    return per_pair * visible_pairs(w, lens) * w.Hq


def gpu_forward_inputs(torch, q, k, v, w, lens, bias=None):
    """float32 forward on the GPU -> O (in q's io type) and natural-log LSE (fp32), rows with no
    key -inf; an additive bias (B, Hq, Sq, Skv) joins the scores after the scale."""
    B, Hq, Sq, _ = q.shape
    group = w.Hq // w.Hkv
    o = torch.empty(B, Hq, Sq, w.Dv, dtype=q.dtype, device=q.device)
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=q.device)
    i = torch.arange(Sq, device=q.device)[:, None]
    j = torch.arange(w.Skv, device=q.device)[None, :]
    for b in range(B):
        L = Sq if lens is None else int(lens[b])
        vis = (i < L) & (j < L)
        if w.causal:
            vis &= j <= i
        if w.window_left >= 0:
            vis &= j >= i - w.window_left
        for h in range(Hq):
            kh = h // group
            kt = k[b, kh].float().t().contiguous()
            s = (q[b, h].float() @ kt) * w.softmax_scale
            if bias is not None:
                s = s + bias[b, h].float()
            s = s.masked_fill(~vis, float("-inf"))
            l = torch.logsumexp(s, dim=-1)
            p = torch.where(vis, torch.exp(s - torch.where(torch.isinf(l), 0.0, l)[:, None]), 0.0)
            o[b, h] = (p @ v[b, kh].float()).to(q.dtype)
            lse[b, h] = l
    return o, lse


COPY_PROBE_BYTES = 1 << 30  # read and written once per launch; 4x the 256 MB Infinity Cache


def copy_probe(torch, dev):
    """A plain fp32 copy (dst = -src, an elementwise kernel no other step of this script launches)
    of COPY_PROBE_BYTES, launched three times: the kernel whose FETCH_SIZE / WRITE_SIZE readings
    calibrate the counters to bytes."""
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def atomic_rate():
    """fp32 atomic adds per second through torch's index_add_ (one atomic per element, consecutive
    lanes on consecutive addresses): the ceiling that bounds a dQ built from fp32 atomics.
    Returns (adds per launch, ms per launch)."""
    import torch
    dev = torch.device("cuda:0")
    n_out, n = 16 << 20, 64 << 20
    out = torch.zeros(n_out, device=dev)
    src = torch.ones(n, device=dev)
    idx = torch.arange(n, device=dev) % n_out
    out.index_add_(0, idx, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        out.index_add_(0, idx, src)
    e1.record()
    torch.cuda.synchronize()
    return n, e0.elapsed_time(e1) / 10


def atomic_probe():
    n, ms = atomic_rate()
    print(json.dumps({"probe": "fp32 atomic add", "adds": n, "ms": round(ms, 4),
                      "g_adds_per_s": round(n / ms / 1e6, 1)}), flush=True)


def kernel_tiles(w, bias=False):
    """The main kernel's head dim and key tile for the workload (32-row q tiles) off the relay
    route: the next native head dim; 256-key tiles (8 waves) up to head dim 192, with an io-type
    bias (the only kind this script draws) up to head dim 128 when S_kv is a multiple of 8, and for
    the QAT variant; else 128-key tiles (4 waves)."""
    kq = next(d for d in (32, 64, 128, 192, 256) if w.Dqk <= d and w.Dv <= (128 if d == 192 else d))
    narrow = kq == 256 or (bias and (kq > 128 or w.Skv % 8 != 0))
    return kq, (128 if narrow else 256), 32


def dq_atomic_adds(w, lens, bias=False):
    """fp32 atomic adds one main-kernel launch makes on the atomic route: every (key tile, q tile)
    pair the mask leaves visible adds a 32-row x kernel-head-dim dQ block, rows past the batch
    entry's query length skipped (the q-tile range rule of the kernel's mask geometry)."""
    kq, bc, br = kernel_tiles(w, bias)
    total = 0
    for b in range(w.B):
        Lq = w.Sq if lens is None else int(lens[b])
        Lkv = w.Skv if lens is None else int(lens[b])
        rows = 0
        for k0 in range(0, Lkv, bc):
            kmax = min(k0 + bc, Lkv) - 1
            qlo = max(k0, 0) if w.causal else 0       # top-left causal: q >= k
            qhi = Lq - 1
            if w.window_left >= 0:
                qhi = min(kmax + w.window_left, qhi)  # window: q <= k + W
            if Lq <= 0 or qlo > qhi:
                continue
            for i in range(qlo // br, qhi // br + 1):
                rows += min(br, Lq - i * br)
        total += rows * w.Hq * kq
    return total


def _pmc_means(directory, counter):
    """Mean per-dispatch value of `counter` for each kernel name in a rocprofv3 --pmc CSV."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {name: (sum(v) / len(v), len(v)) for name, v in out.items()}


def write_traffic_record(workload, det_arg, dtype, fetch_dir, write_dir):
    import attention_backward_sdpa_amd as lib
    w = synth.WORKLOADS[workload]
    det = int(w.deterministic) if det_arg < 0 else det_arg
    rec = {"kernel_source_hash": kernel_source_hash(), "workload": w.name,
           "dq_route": lib.dq_route(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, det), "dtype": dtype,
           "copy_probe_bytes": COPY_PROBE_BYTES}
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        means = _pmc_means(d, counter)
        main = [(n, v) for n, v in means.items() if "bwd_main_kernel" in n]
        copy = [(n, v) for n, v in means.items() if "neg_kernel" in n]
        if len(main) != 1 or len(copy) != 1:
            raise SystemExit(f"{d}: expected one main kernel and one copy-probe kernel for "
                             f"{counter}, found {len(main)} and {len(copy)}")
        main_kib, n_main = main[0][1]
        copy_kib, n_copy = copy[0][1]
        factor = (COPY_PROBE_BYTES / 1024.0) / copy_kib  # true KiB per counted KiB
        bytes_ = main_kib * factor * 1024.0
        rec[counter] = {"main_kib_per_dispatch": main_kib, "main_dispatches": n_main,
                        "copy_kib_per_dispatch": copy_kib, "copy_dispatches": n_copy,
                        "scale_factor": factor, "main_bytes_per_launch": bytes_,
                        "kernel": main[0][0]}
        total += bytes_
    rec["hbm_bytes_per_launch"] = total
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, inp, lens, dtype="bf16", budget_s=15.0, qat=False):
    """The fp64 CPU oracle (unchanged) on the first query heads of batch entry 0, timed until
    about budget_s seconds of work; the rate is scaled to the same FLOP convention.  `cores` is
    the thread count of the BLAS pool the oracle ran on, `cores_available` the CPUs this process
    may run on (sched_getaffinity)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = os.cpu_count()
    group = w.Hq // w.Hkv
    f = lambda x: synth.bits_to_f32(x, dtype).astype(np.float64)
    to_io = synth.fp16_bits if dtype == "fp16" else synth.bf16_bits
    L = None if lens is None else [int(lens[0])]
    flops = done = 0.0
    heads = 0
    t_total = 0.0
    while heads < w.Hq and t_total < budget_s:
        h = heads
        kh = h // group
        sl = lambda a, hh: a[0:1, hh:hh + 1]
        q, kk, vv, do = f(sl(inp.q, h)), f(sl(inp.k, kh)), f(sl(inp.v, kh)), f(sl(inp.do, h))
        o, lse = oracle.forward(q, kk, vv, w.softmax_scale, causal=w.causal,
                                window_left=w.window_left, seq_q_lens=L, seq_kv_lens=L)
        o = f(to_io(o.astype(np.float32)))
        lse = lse.astype(np.float32).astype(np.float64)
        t0 = time.perf_counter()
        if qat:
            oracle.qat_backward(q, kk, vv, o, do, lse, w.softmax_scale, causal=w.causal)
        else:
            oracle.backward(q, kk, vv, o, do, lse, w.softmax_scale, causal=w.causal,
                            window_left=w.window_left, seq_q_lens=L, seq_kv_lens=L)
        t_total += time.perf_counter() - t0
        one = synth.small_variant(w, B=1, Hq=1, Hkv=1)
        flops += algorithmic_flops(one, None if lens is None else [lens[0]])
        heads += 1
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "cores_available": int(affinity), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.Hq} (batch, query-head) slices of {w.name}, "
                      f"{'NVFP4-QAT ' if qat else ''}backward only, fp64 numpy, {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_causal_s4096_d128", choices=list(synth.WORKLOADS))
    ap.add_argument("--deterministic", type=int, default=-1,
                    help="override the workload's dQ route (-1: as the workload states; 0 fp32 "
                         "atomics, 1 deterministic (the library's choice), 2 dS panels + dq2k, "
                         "3 dQ partials + ordered reduction, 4 ordered relay)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"],
                    help="io element type of Q, K, V, O, dO and the gradients")
    ap.add_argument("--bias", default="none", choices=["none", "bias", "dbias", "dbias_io"],
                    help="add a per-batch additive bias (B, Hq, Sq, Skv) of the io type, drawn "
                         "N(0,1) (bias), and also produce its gradient in fp32 (dbias) or in the "
                         "io type (dbias_io)")
    ap.add_argument("--qat", action="store_true",
                    help="the NVFP4 attention-QAT backward (sdpa_bwd_nvfp4_qat) on the workload's "
                         "shape (MHA, head dim 128, no window or padding); O and LSE come from the "
                         "forward on the unquantised inputs, which changes no timed work")
    ap.add_argument("--dims", default=None, metavar="DQK,DV",
                    help="override the workload's head dims (multiples of 8 up to 256, DV <= DQK: "
                         "other than the native pairs they run on the next native kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run a plain 1 GiB fp32 copy kernel three times "
                         "(the calibration kernel of the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--atomic-probe", action="store_true",
                    help="measure the device's fp32 atomic-add rate (torch index_add_, 64 Mi "
                         "coalesced adds into 16 Mi floats) and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: read two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) "
                         "of a --copy-probe run and write the main kernel's HBM traffic record")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_record(args.workload, args.deterministic, args.dtype, *args.traffic_from)
        return
    if args.atomic_probe:
        atomic_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              f"attention backward shards over (batch, KV-head group) with no communication, "
              f"so the whole-job rate is N times the one-GPU rate).", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_backward_sdpa_amd as lib

    w = synth.WORKLOADS[args.workload]
    if args.dims:
        dqk, dv = (int(x) for x in args.dims.split(","))
        w = synth.small_variant(w, Dqk=dqk, Dv=dv, name=f"{w.name}_dims{dqk}x{dv}")
    det = int(w.deterministic) if args.deterministic < 0 else args.deterministic
    route = lib.dq_route(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, det)
    if route < 0:
        raise SystemExit(f"--deterministic {det}: not a dQ route")
    inp = synth.draw_inputs(w, dtype=args.dtype)
    lens = inp.seq_q_lens
    dev = torch.device("cuda:0")
    io = torch.float16 if args.dtype == "fp16" else torch.bfloat16
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(io).to(dev)
    q, k, v, do = bf(inp.q), bf(inp.k), bf(inp.v), bf(inp.do)
    bias = dbias = None
    if args.bias != "none":
        gen = torch.Generator(device=dev).manual_seed(1000)
        bias = torch.randn(w.B, w.Hq, w.Sq, w.Skv, generator=gen, device=dev).to(io)
        if args.bias in ("dbias", "dbias_io"):
            dbias = torch.empty(w.B, w.Hq, w.Sq, w.Skv, device=dev,
                                dtype=torch.float32 if args.bias == "dbias" else io)
    if args.qat and (w.Hq != w.Hkv or w.Dqk != 128 or w.Dv != 128 or w.window_left >= 0 or
                     lens is not None or args.bias != "none" or args.dtype != "bf16"):
        raise SystemExit("--qat: MHA, head dim 128, bf16, no window, padding or bias")
    o, lse = gpu_forward_inputs(torch, q, k, v, w, lens, bias)
    lens_t = None if lens is None else torch.from_numpy(lens).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
              deterministic=det, seq_q_lens=lens_t, seq_kv_lens=lens_t, bias=bias, dbias=dbias)
    nws = (lib.nvfp4_qat_workspace_size(w.B, w.Hq, w.Sq, w.Skv, 128, w.causal, det) if args.qat
           else lib.run_workspace_size(q, k, v, **kw))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        if args.qat:
            lib.sdpa_bwd_nvfp4_qat(q, k, v, o, do, lse, dq, dk, dv, scale=w.softmax_scale,
                                   causal=w.causal, deterministic=det, workspace=ws, stream=stream,
                                   events=events)
        elif bias is None:
            lib.sdpa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale=w.softmax_scale,
                            causal=w.causal, window_left=w.window_left, deterministic=det,
                            seq_q_lens=lens_t, seq_kv_lens=lens_t, workspace=ws, stream=stream,
                            events=events)
        else:
            lib.sdpa_bwd_run(q, k, v, o, do, lse, dq, dk, dv, workspace=ws, stream=stream,
                             events=events, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def make_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n)]
        for row in evs:
            for e in row:
                e.record(stream)  # materialise the underlying hipEvent
        return evs

    # Timed region: the library records HIP events on the launch stream around the main kernel
    # only (the roofline's launch duration); every other event slot is left out, so the step
    # time carries no extra stream packets.
    evs = make_events(args.steps)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        step([None, evs[s][1], evs[s][2], None, None])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    main_ms = float(np.mean([row[1].elapsed_time(row[2]) for row in evs]))
    # Per-stage breakdown from a second, untimed pass with all five events.
    evs = make_events(args.steps)
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    stage_avg = np.array([[row[i].elapsed_time(row[i + 1]) for i in range(4)] for row in evs]).mean(axis=0)

    flops = algorithmic_flops(w, lens)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # on the dS-panel route the main kernel skips GEMM4 (dQ = dS K), which dq2k performs
    main_flops = flops * ((2 * w.Dqk + 2 * w.Dv) / (3 * w.Dqk + 2 * w.Dv)
                          if route == lib.DQ_DS_PANELS else 1.0)
    main_tflops = main_flops / (main_ms * 1e-3) / 1e12
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash() and t.get("workload") == w.name \
                and t.get("dq_route") == route and t.get("dtype", "bf16") == args.dtype \
                and args.bias == "none":
            traffic = t["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Skv": w.Skv, "Dqk": w.Dqk, "Dv": w.Dv, "causal": w.causal,
                   "window_left": w.window_left, "padded": w.padded,
                   "dq_route": ROUTE_NAMES[route],
                   "nvfp4_qat": bool(args.qat),
                   "bias": {"none": "none", "bias": f"{args.dtype} (B, Hq, Sq, Skv)",
                            "dbias": f"{args.dtype} (B, Hq, Sq, Skv) with fp32 dBias",
                            "dbias_io": f"{args.dtype} (B, Hq, Sq, Skv) with {args.dtype} dBias"}[args.bias],
                   "algorithmic_gflop": round(flops / 1e9, 3)},
        "stage_ms": {"preprocess": round(float(stage_avg[0]), 4), "main": round(float(stage_avg[1]), 4),
                     "gqa_reduce": round(float(stage_avg[2]), 4),
                     ROUTE_STAGE[route]: round(float(stage_avg[3]), 4)},
        "roofline": {"kernel": "bwd_main_kernel", "bound": "mfma",
                     "achieved": round(main_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(main_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if route == lib.DQ_ATOMIC:
        # the rate at which the main kernel's fp32 dQ atomics retire, next to the rate of a kernel
        # that does nothing but fp32 atomic adds (torch's index_add_), measured now
        adds = dq_atomic_adds(w, lens, args.bias != "none")
        n, ms = atomic_rate()
        achieved = adds / (main_ms * 1e-3)
        probe = n / (ms * 1e-3)
        out["dq_atomics"] = {"adds_per_launch": adds, "main_us": round(main_ms * 1e3, 1),
                             "achieved_g_adds_per_s": round(achieved / 1e9, 1),
                             "probe_g_adds_per_s": round(probe / 1e9, 1),
                             "achieved_over_probe": round(achieved / probe, 3)}
    if args.copy_probe:
        copy_probe(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, lens, args.dtype, qat=args.qat)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
