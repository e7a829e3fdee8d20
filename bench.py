"""Benchmark of the block-scaled FP8 GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the whole hot path, fp8_block_gemm_ex (dispatcher +
kernel, with split-K's fixed-order reduction inside the kernel), on one
batch of synthetic input of the named workload (default: the prefill shape
M=16384, N=4096, K=4096, bf16 output, the largest configuration of the
metric; its N=1 line is the headline).  Inputs sit in HBM before timing
starts.  Steps rotate over input copies such that between two uses of a copy
the others move at least 2x the 256 MB MALL, and a scrub pass over 1 GiB of
other memory separates the untimed steps from the timed ones, so every timed
step reads its operands from HBM (step_schedule gives the exact order).
Steps are issued from HIP graphs (captured through torch; one graph holds
every timed step) so that host launch cost does not hide the GPU time of a
microsecond-scale kernel.  The
timed region is bracketed by device synchronisation and by HIP events on the
stream the kernels run on; ms_per_step and the roofline's per-launch
duration come from those events.

Prints ONE JSON line (the benchmark contract).  Its per_config key holds the
metric's other configurations (the small, decode, short-K and mid-M shapes,
the prefill shape with fp32 output, and the plain entry point fp8_block_gemm
on the decode shape), each timed the same way; on rank 0 at N=1 it also
carries the CPU oracle timed on a bounded sample of the same workload.

Other modes (for profiles):
  --sweep FILE        every workload and sweep point, one JSON line each, to FILE
  --dispatch-sweep FILE   the dispatcher's choice against every forced alternative
                      on the pages' (M, N, K) shape sets, one JSON line per shape
  --floors FILE       platform floors: a one-element kernel's launch-to-launch time
                      in graph replays, and device copies of 0.25-256 MiB
  --copy-bytes B      only a plain device copy of B bytes (calibrates HBM counters)
  --probe-load FILE   the load-path probe (libfp8bg_probe.so): one workgroup per CU
                      streaming 1 MiB from a shared 256 KiB region (L2 hits) or its
                      own 1 MiB region (HBM), 4 or 8 waves, direct-to-LDS or register
                      loads, 8 KB in flight per wave; one JSON line per case to FILE
  --op quantize       time the per-token 1x128 activation quantiser (bf16 -> E4M3
                      codes + fp32 scales) on the workload's A shape instead
  --op quantize_weights   the 128x128 weight-block quantiser on the workload's B shape
  --op grouped        the grouped (mixture-of-experts) GEMM on --moe NAME (default:
                      64 tokens routed top-8 over 256 experts of 512 x 4096)
  --no-graph          launch each step eagerly (for counter collection)
  --no-per-config     only the named workload
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
MALL_BYTES = 256 << 20
METRIC = "TFLOP/s and % of roofline (HBM or FP8 MFMA) per (M,N,K), 1×MI355X"


KERNEL_SOURCES = ["block_scaled_fp8_gemm_amd/csrc/fp8bg_kernels.hip", "block_scaled_fp8_gemm_amd/csrc/fp8bg_device.hpp",
                  "block_scaled_fp8_gemm_amd/csrc/fp8bg_configs.h"]


def kernel_source_hash():
    """Hash of the kernel sources' code (comments and whitespace removed, so a
    comment edit does not invalidate a committed traffic profile)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_record(workload, out="bf16"):
    """The machine-readable record of the committed FETCH_SIZE / WRITE_SIZE
    profile of `workload` with output dtype `out`, or None (a profile file
    holds one record per output dtype it covers)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_record:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("out") == out:
                return rec
    return None


def profiled_traffic(workload, plan, out):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE profile
    of this workload, if that profile was taken on the same kernel sources and
    the same plan; else None."""
    rec = traffic_record(workload, out)
    if rec is None:
        return None
    same = (rec.get("source_hash") == kernel_source_hash() and rec.get("variant") == plan["variant_name"]
            and rec.get("config") == plan["config"] and rec.get("split_k") == plan["split_k"]
            and rec.get("out") == out)
    return rec["traffic_bytes"] if same else None


def alg_bytes(M, N, K, out_bytes):
    """Each input read once, C written once (split-K partials are overhead)."""
    G, NB = K // 128, (N + 127) // 128
    return M * K + N * K + 4 * M * G + 4 * NB * G + M * N * out_bytes


def make_device_copies(w, M, copies, torch, W):
    d = W.make_workload(w, M)
    dev = torch.device("cuda:0")
    base = {
        "A": torch.from_numpy(d["A"]).to(dev).view(torch.float8_e4m3fn),
        "a_s": torch.from_numpy(d["a_s"]).to(dev),
        "B": torch.from_numpy(d["B"]).to(dev).view(torch.float8_e4m3fn),
        "b_s": torch.from_numpy(d["b_s"]).to(dev),
    }
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    return d, sets


def copies_for(per_copy, cap):
    """Input copies to rotate over: enough that between two uses of one copy
    the other copies move at least 2x the MALL (so every use reads HBM), at
    most `cap`, at least 2."""
    return max(2, min(cap, -(-2 * MALL_BYTES // per_copy) + 1))


GRAPH_MAX_STEPS = 4096


def chunk_sizes(steps, copies):
    """The timed steps as graph replays: one graph of all steps while they
    number at most GRAPH_MAX_STEPS (or one pass over the copies, if that is
    longer), the last one shorter; they add up to `steps`.  Inside a graph
    the launches run back to back; each further replay would add a gap of
    ~9 us (kernel traces) that is no part of the kernel."""
    chunk = max(1, min(steps, max(copies, GRAPH_MAX_STEPS)))
    return [chunk] * (steps // chunk) + ([steps % chunk] if steps % chunk else [])


def step_schedule(copies, steps, warmup, use_graph):
    """The order in which time_steps touches the input copies, as a list of
    (phase, copy) pairs: phase "warm" (eager warm-up steps), "replay" (one
    untimed replay of each captured graph, the case where a graph cannot be
    uploaded instead), "scrub" (a pass over SCRUB_BYTES
    of other memory, copy None) and "timed".  Pure; the CPU tests check on it
    that every timed use of a copy comes at least 2x the MALL after its last
    earlier use."""
    ev = [("warm", i % copies) for i in range(warmup)]
    if use_graph:
        sizes = chunk_sizes(steps, copies)
        for n in sorted(set(sizes)):
            ev += [("replay", i) for i in range(n)]
        ev.append(("scrub", None))
        for n in sizes:
            ev += [("timed", i) for i in range(n)]
    else:
        ev.append(("scrub", None))
        ev += [("timed", i % copies) for i in range(steps)]
    return ev


SCRUB_BYTES = 4 * MALL_BYTES   # bytes a scrub pass moves (half read, half written)
_scrub_bufs = []


def scrub_mall(stream, torch):
    """Evicts the MALL and the L2s: one device copy moving SCRUB_BYTES of
    memory no step uses, on `stream`, then a device synchronisation."""
    if not _scrub_bufs:
        half = SCRUB_BYTES // 2
        _scrub_bufs.extend([torch.ones(half, dtype=torch.uint8, device="cuda:0"),
                            torch.empty(half, dtype=torch.uint8, device="cuda:0")])
    with torch.cuda.stream(stream):
        _scrub_bufs[1].copy_(_scrub_bufs[0], non_blocking=True)
    torch.cuda.synchronize()


def upload_graph(graph, stream):
    """hipGraphUpload of a captured graph, so that its first launch does not
    pay the upload; False where that cannot be done (the caller then replays
    the graph once, untimed)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        f = hip.hipGraphUpload
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        ex = graph.raw_cuda_graph_exec()
    except (OSError, AttributeError, RuntimeError):
        return False
    return bool(ex) and f(ctypes.c_void_p(ex), ctypes.c_void_p(stream.cuda_stream)) == 0


def time_steps(step, copies, steps, warmup, use_graph, stream, torch):
    """Runs `warmup` untimed steps, then times exactly `steps` steps with HIP
    events on `stream`, in the order step_schedule gives: replayed from HIP
    graphs (chunk_sizes; each graph uploaded first, or where that is not
    available replayed once, untimed) unless use_graph is false, and
    preceded by a MALL scrub
    so that no timed step finds its inputs in a cache.  Returns (GPU ms,
    wall seconds)."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()

    plan_seq = []
    if use_graph:
        sizes = chunk_sizes(steps, copies)
        graphs = {}
        for n in sorted(set(sizes)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    step(i)
            graphs[n] = g
        plan_seq = [graphs[n] for n in sizes]
        with torch.cuda.stream(stream):   # replay() launches on the current stream
            for n in sorted(graphs):      # uploaded, else replayed once untimed
                if not upload_graph(graphs[n], stream):
                    graphs[n].replay()
        torch.cuda.synchronize()
    scrub_mall(stream, torch)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if use_graph:
            for g in plan_seq:
                g.replay()
        else:
            for i in range(steps):
                step(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1), wall


def run_workload(args, w, M, out_name, torch, fbg, W, steps, warmup, use_graph=True,
                 variant="auto", split_k=0, cfg=None, entry="ex", max_copies=None):
    """Times `steps` GEMM calls on workload `w` at M rows.  entry "ex":
    fp8_block_gemm_ex with a caller workspace (variant / split_k / cfg may
    force a kernel); entry "fp8_block_gemm": the plain entry point with no
    workspace, as a caller without one uses it."""
    out_dtype = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[out_name]
    out_bytes = 4 if out_name == "fp32" else 2
    N, K = w.N, w.K
    per_copy = M * K + N * K + 4 * M * (K // 128) + 4 * ((N + 127) // 128) * (K // 128) + M * N * out_bytes
    copies = copies_for(per_copy, max_copies or args.max_copies)
    d, sets = make_device_copies(w, M, copies, torch, W)
    outs = [torch.empty((M, N), dtype=out_dtype, device="cuda:0") for _ in range(copies)]
    if cfg is not None:
        os.environ["FBG_FORCE_CONFIG"] = str(cfg)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if entry == "fp8_block_gemm":
        assert variant == "auto" and split_k == 0 and cfg is None
        plan = fbg.plan(M, N, K, out_dtype, cu, "auto", 1)   # no workspace: the unsplit plan
        ws = "library"
    else:
        plan = fbg.plan(M, N, K, out_dtype, cu, variant, split_k)
        ws = torch.zeros(max(fbg.workspace_size(M, N, K, variant, split_k), 16), dtype=torch.uint8,
                         device="cuda:0")
    if cfg is not None:
        plan["config"] = cfg
    stream = torch.cuda.Stream()

    def step(i):
        s = sets[i % copies]
        fbg.gemm(s["A"], s["a_s"], s["B"], s["b_s"], out_dtype=out_dtype, out=outs[i % copies],
                 workspace=ws, stream=stream, variant=variant, split_k=split_k)

    gpu_ms, wall = time_steps(step, copies, steps, warmup, use_graph, stream, torch)
    ms_per_step = gpu_ms / steps
    flops = 2 * M * N * K
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    nbytes = alg_bytes(M, N, K, out_bytes)
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    bound = "hbm" if flops / nbytes < FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP8_PEAK_TFLOPS, 4)}
    if cfg is not None:
        os.environ.pop("FBG_FORCE_CONFIG", None)
    return {"d": d, "plan": plan, "ms_per_step": ms_per_step, "tflops": tflops, "gbs": gbs, "roof": roof,
            "copies": copies, "wall_s": wall, "alg_bytes": nbytes}


def quantize_bytes(M, K):
    """Algorithmic bytes of the activation quantiser: bf16 x read once, E4M3 A
    and fp32 a_s written once."""
    return 2 * M * K + M * K + 4 * M * (K // 128)


def activation_bits(M, K, seed, outlier_frac, np):
    """Seeded bf16 activations of the workload recipe (N(0,1), outlier rows x10)."""
    import torch
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(M, K)).astype(np.float32)
    if outlier_frac:
        x[rng.random(M) < outlier_frac] *= 10.0
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run_quantize(args, w, M, torch, fbg, steps, warmup, use_graph=True, weights=False):
    """Times the activation quantiser on the workload's A [M,K] or, with
    weights=True, the 128x128 weight quantiser on its B [N,K]."""
    import numpy as np
    K = w.K
    if weights:
        M = w.N
        rng = np.random.default_rng(w.seed + 1000)
        wf = (rng.normal(size=(M, K)) * 0.02).astype(np.float32)
        bits = torch.from_numpy(wf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nbytes = 2 * M * K + M * K + 4 * ((M + 127) // 128) * (K // 128)
        srows = (M + 127) // 128
    else:
        bits = activation_bits(M, K, w.seed, w.outlier_frac, np)
        nbytes = quantize_bytes(M, K)
        srows = M
    copies = copies_for(nbytes, args.max_copies)
    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    As = [torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(copies)]
    ss = [torch.empty((srows, K // 128), dtype=torch.float32, device=dev) for _ in range(copies)]
    stream = torch.cuda.Stream()
    fn = fbg.quantize_blocks if weights else fbg.quantize_rows

    def step(i):
        j = i % copies
        fn(xs[j], As[j], ss[j], stream=stream)

    gpu_ms, wall = time_steps(step, copies, steps, warmup, use_graph, stream, torch)
    ms = gpu_ms / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return {"bits": bits, "ms_per_step": ms, "gbs": gbs, "roof": roof, "copies": copies, "alg_bytes": nbytes,
            "rows": M}


def grouped_alg_bytes(d, out_bytes):
    """A, a_s, the weights and scales of the experts that hold rows (the
    others are never read), the offsets and C, each once."""
    counts = d["offsets"][1:] - d["offsets"][:-1]
    active = int((counts > 0).sum())
    E, N, K = d["B"].shape
    M, G = d["A"].shape[0], K // 128
    return M * K + 4 * M * G + active * (N * K + 4 * ((N + 127) // 128) * G) + 4 * (E + 1) + M * N * out_bytes


def run_probe_load(path, torch):
    """The load-path probe: per-CU streaming rate of one workgroup per CU."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_scaled_fp8_gemm_amd", "libfp8bg_probe.so"))
    f = lib.fbg_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    per_wg = 1 << 20
    shared = torch.zeros(256 << 10, dtype=torch.uint8, device=dev)
    # two sets of private regions, used in turn: 2 x 256 MiB > the MALL
    private = [torch.zeros(cu * per_wg, dtype=torch.uint8, device=dev) for _ in range(2)]
    sink = torch.zeros(cu * 64 * 8, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    reps = 20
    with open(path, "w") as fh:
        for src_name in ("l2_shared_256KiB", "hbm_private_1MiB"):
            for waves in (4, 8):
                for dma in (1, 0):
                    loads = per_wg // (waves * 1024)

                    def launch(i):
                        buf = shared if src_name.startswith("l2") else private[i % 2]
                        stride = 0 if src_name.startswith("l2") else per_wg
                        region = shared.numel() if src_name.startswith("l2") else per_wg
                        st = f(buf.data_ptr(), buf.numel(), stride, region, cu, waves, dma, loads, sink.data_ptr(),
                               ctypes.c_void_p(stream.cuda_stream))
                        if st != 0:
                            raise RuntimeError(f"fbg_probe_stream returned {st}")

                    with torch.cuda.stream(stream):
                        for i in range(4):
                            launch(i)
                        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        t0.record(stream)
                        for i in range(reps):
                            launch(i)
                        t1.record(stream)
                    torch.cuda.synchronize()
                    us = t0.elapsed_time(t1) * 1e3 / reps
                    line = {"probe": "load_path", "source": src_name, "waves": waves,
                            "loads": "direct-to-LDS" if dma else "registers", "workgroups": cu,
                            "bytes_per_workgroup": per_wg, "us": round(us, 2),
                            "gbs_per_cu": round(per_wg / us / 1e3, 1), "tbs_total": round(cu * per_wg / us / 1e6, 2)}
                    fh.write(json.dumps(line) + "\n")
                    print(json.dumps(line), flush=True)


def run_grouped(args, mw, torch, fbg, W, steps, warmup, use_graph=True, out_name="bf16"):
    """Times fp8_block_gemm_grouped on the MoE workload `mw`, rotating over
    input copies (at least two: the weights alone exceed the MALL)."""
    import numpy as np
    out_dtype = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[out_name]
    out_bytes = 4 if out_name == "fp32" else 2
    d = W.make_moe_workload(mw)
    dev = torch.device("cuda:0")
    base = {
        "A": torch.from_numpy(d["A"]).to(dev).view(torch.float8_e4m3fn),
        "a_s": torch.from_numpy(d["a_s"]).to(dev),
        "B": torch.from_numpy(d["B"]).to(dev).view(torch.float8_e4m3fn),
        "b_s": torch.from_numpy(d["b_s"]).to(dev),
        "offsets": torch.from_numpy(d["offsets"].astype(np.int32)).to(dev),
    }
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    copies = copies_for(per_copy, args.max_copies)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    M, N = d["A"].shape[0], d["B"].shape[1]
    outs = [torch.empty((M, N), dtype=out_dtype, device=dev) for _ in range(copies)]
    stream = torch.cuda.Stream()
    if args.cfg is not None:
        os.environ["FBG_FORCE_CONFIG"] = str(args.cfg)

    def step(i):
        s = sets[i % copies]
        fbg.grouped_gemm(s["A"], s["a_s"], s["B"], s["b_s"], s["offsets"], out_dtype=out_dtype,
                         out=outs[i % copies], stream=stream)

    gpu_ms, wall = time_steps(step, copies, steps, warmup, use_graph, stream, torch)
    os.environ.pop("FBG_FORCE_CONFIG", None)
    ms = gpu_ms / steps
    nbytes = grouped_alg_bytes(d, out_bytes)
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = 2 * M * N * d["A"].shape[1]
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}
    cfg = args.cfg if args.cfg is not None else fbg.grouped_plan(mw.experts, M, N, d["A"].shape[1])["config"]
    return {"d": d, "ms_per_step": ms, "gbs": gbs, "tflops": flops / (ms * 1e-3) / 1e12, "roof": roof,
            "copies": copies, "alg_bytes": nbytes, "M": M, "N": N, "flops": flops, "cfg": cfg}


def cpu_baseline_grouped(d, flops_per_call, budget_s=12.0):
    """The oracle's grouped GEMM over the full MoE workload, repeated until
    about `budget_s` have passed."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.grouped_gemm(d["A"], d["a_s"], d["B"], d["b_s"], d["offsets"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": round(reps * flops_per_call / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"full MoE workload (fp64 oracle, every expert's GEMM) repeated {reps}x in {el:.1f} s"}


def cpu_baseline_quantize(bits, budget_s=12.0, weights=False):
    """The oracle's row (or weight-block) quantiser, on the host's cores, over
    the full input repeated until about `budget_s` have passed."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    R, K = bits.shape
    nbytes = 3 * R * K + 4 * ((R + 127) // 128 if weights else R) * (K // 128)
    fn = oracle.quantize_blocks if weights else oracle.quantize_rows
    while True:
        fn(bits)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": round(reps * nbytes / el / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"full {'weight' if weights else 'activation'} matrix quantised {reps}x in {el:.1f} s"}


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, budget_s=12.0, single_budget_s=4.0, max_flops_per_call=20e9):
    """The oracle as it stands, on the host's cores, repeated over the
    workload until about `budget_s` has passed; then once more on one thread
    for about `single_budget_s`.  A workload of more than `max_flops_per_call`
    (the prefill shape: 550 GFLOP, over an hour for the fp64 oracle) is
    sampled: the oracle computes its first rows only (every column, the whole
    K), as many as fit in that bound; the rate is the same per row."""
    import oracle
    A, a_s, B, b_s = d["A"], d["a_s"], d["B"], d["b_s"]
    M, K = A.shape
    N = B.shape[0]
    rows = M
    if 2 * M * N * K > max_flops_per_call:
        rows = max(1, int(max_flops_per_call // (2 * N * K)))
        rows = 1 << (rows.bit_length() - 1)      # a power of two
        A, a_s = A[:rows], a_s[:rows]
    flops_per_call = 2 * rows * N * K
    oracle.block_gemm(A[:1], a_s[:1], B, b_s)  # load the library

    def timed(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.block_gemm(A, a_s, B, b_s)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 20000:
                return reps, el

    cores = oracle.threads()
    reps, el = timed(budget_s)
    oracle.set_threads(1)
    reps1, el1 = timed(single_budget_s)
    oracle.set_threads(cores)
    what = "full workload GEMM" if rows == M else f"rows 0..{rows - 1} of the workload (all {N} columns, K={K})"
    return {"value": round(reps * flops_per_call / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{what} (fp64 oracle, E4M3 decode) repeated {reps}x in {el:.1f} s",
            "value_1_thread": round(reps1 * flops_per_call / el1 / 1e12, 6), "cpu": host_cpu_model()}


def dispatch_sweep(path, torch, fbg, steps=100, warmup=10):
    """Dispatcher evidence: on every (M, N, K) of the pages' shape sets
    (N in {512, 1536, 4096, 8192}, K in {256, 1024, 4096}, M from 1 to 4096),
    times the dispatcher's own choice and every forced alternative (each
    generic tile, the main swap-AB tiles with and without split-K, the short-K
    tiles at K = 256) the same way as the benchmark (HIP-graph replays over
    input copies rotated past the MALL), one JSON line per shape with the
    regret of the dispatcher's choice against the fastest other choice.  The
    operands are random non-NaN E4M3 bytes and random scales made on the GPU
    (timing only, no parity)."""
    dev = torch.device("cuda:0")
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    def codes(rows, cols):
        c = torch.randint(0, 254, (rows, cols), device=dev, generator=gen, dtype=torch.int32)
        return (c + (c >= 0x7F).int()).to(torch.uint8).view(torch.float8_e4m3fn)

    with open(path, "w") as f:
        for N in (512, 1536, 4096, 8192):
            for K in (256, 1024, 4096):
                for M in (1, 16, 32, 64, 128, 256, 512, 1024, 4096):
                    G, NB = K // 128, (N + 127) // 128
                    per_copy = M * K + N * K + 4 * M * G + 4 * NB * G + 2 * M * N
                    copies = copies_for(per_copy, 256)
                    base = {"A": codes(M, K), "B": codes(N, K),
                            "a_s": torch.rand((M, G), device=dev, generator=gen) * 0.01 + 1e-3,
                            "b_s": torch.rand((NB, G), device=dev, generator=gen) * 0.01 + 1e-3}
                    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
                    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
                    cands = [("auto", None)] + [("generic", c) for c in range(12)]
                    cands += [(v, c) for v in ("swap_ab", "swap_ab_splitk") for c in (2, 4, 7, 12, 19, 22)]
                    cands += [("swap_ab", 23)]   # 8-row tiles never split
                    if K == 256:
                        cands += [("short_k256", c) for c in range(16)]
                    cands += [("auto", None)]   # timed first and last: the faster of the two counts
                    res = {}
                    for variant, cfg in cands:
                        p = fbg.plan(M, N, K, torch.bfloat16, cu, variant, 0) if cfg is None else None
                        if cfg is not None:
                            os.environ["FBG_FORCE_CONFIG"] = str(cfg)
                        ws = torch.zeros(max(fbg.workspace_size(M, N, K, variant, 0), 16), dtype=torch.uint8,
                                         device=dev)
                        stream = torch.cuda.Stream()

                        def step(i):
                            t = sets[i % copies]
                            fbg.gemm(t["A"], t["a_s"], t["B"], t["b_s"], out=outs[i % copies], workspace=ws,
                                     stream=stream, variant=variant)

                        try:
                            ms, _ = time_steps(step, copies, steps, warmup, True, stream, torch)
                            t_us = ms / steps * 1e3
                            res[(variant, cfg)] = min(t_us, res.get((variant, cfg), t_us))
                        except fbg.FP8BGError:
                            pass
                        finally:
                            os.environ.pop("FBG_FORCE_CONFIG", None)
                        if cfg is None:
                            auto_plan = p
                    # An unsplit automatic plan is the same launch as its own
                    # configuration forced: the three timings of that launch
                    # are pooled, and the regret is taken against the fastest
                    # other choice (negative: the choice beats them all).
                    auto_us = res[("auto", None)]
                    own = None
                    if auto_plan["split_k"] == 1 and auto_plan["variant_name"] != "swap_ab_splitk":
                        own = (auto_plan["variant_name"], auto_plan["config"])
                        auto_us = min(auto_us, res.get(own, auto_us))
                    best = min((v for v in res.items() if v[0][0] != "auto" and v[0] != own), key=lambda kv: kv[1])
                    line = {"M": M, "N": N, "K": K, "auto": {"variant": auto_plan["variant_name"],
                                                              "cfg": auto_plan["config"],
                                                              "split_k": auto_plan["split_k"],
                                                              "us": round(auto_us, 3)},
                            "best": {"variant": best[0][0], "cfg": best[0][1], "us": round(best[1], 3)},
                            "regret": round(auto_us / best[1] - 1.0, 4),
                            "all": {f"{v}:{c}": round(t, 3) for (v, c), t in res.items()}}
                    f.write(json.dumps(line) + "\n")
                    f.flush()
                    print(json.dumps({k: line[k] for k in ("M", "N", "K", "auto", "best", "regret")}), flush=True)
                    del sets, outs, base


def copy_floor_us(nbytes, torch, steps=200, warmup=20):
    """The same-bytes floor of a launch on this GPU: a device-to-device copy
    that reads nbytes/2 and writes nbytes/2, timed like the kernels (HIP-graph
    replays, buffers rotated past the MALL).  Returns microseconds per copy."""
    half = max(16, (nbytes // 2 + 15) // 16 * 16)
    copies = copies_for(2 * half, 256)
    src = [torch.empty(half, dtype=torch.uint8, device="cuda:0").fill_(1) for _ in range(copies)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
    stream = torch.cuda.Stream()

    def step(i):
        dst[i % copies].copy_(src[i % copies], non_blocking=True)

    ms, _ = time_steps(step, copies, steps, warmup, True, stream, torch)
    return ms / steps * 1e3


def platform_floors(path, torch):
    """Launch and streaming floors of this GPU, timed like the kernels
    (HIP-graph replays, buffers rotated past the MALL, scrubbed first): a
    one-element fill (the launch-to-launch time of a kernel that does no
    work), device copies of 0.25 .. 256 MiB read + as many written, and the
    platform library's FP8 GEMM on the prefill shape."""
    lines = []
    one = [torch.empty(1, dtype=torch.float32, device="cuda:0") for _ in range(2000)]
    stream = torch.cuda.Stream()
    ms, _ = time_steps(lambda i: one[i].fill_(1.0), 2000, 2000, 100, True, stream, torch)
    lines.append({"floor": "launch", "what": "one-element fill kernel, 2000 back to back in one HIP graph",
                  "us": round(ms / 2000 * 1e3, 3)})
    for mib in (0.25, 1, 2, 8, 64, 256):
        nbytes = int(2 * mib * (1 << 20))
        us = copy_floor_us(nbytes, torch, steps=200 if mib < 64 else 20, warmup=10)
        lines.append({"floor": "copy", "read_bytes": nbytes // 2, "written_bytes": nbytes // 2,
                      "us": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)})
    lines += library_fp8_gemm(torch)
    with open(path, "w") as f:
        for line in lines:
            f.write(json.dumps(line) + "\n")
            print(json.dumps(line), flush=True)


def library_fp8_gemm(torch, M=16384, N=4096, K=4096, steps=20):
    """The platform library's FP8 GEMM (hipBLASLt through torch._scaled_mm,
    bf16 output) on the prefill shape, timed like the kernels: a reference
    point for the MFMA-bound kernel.  It applies one scale per tensor, or one
    per row of A and per column of B -- not the 1x128 / 128x128 block scales,
    so it does less work than the block-scaled GEMM."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)

    def codes(rows, cols):
        c = torch.randint(0, 254, (rows, cols), device=dev, generator=gen, dtype=torch.int32)
        return (c + (c >= 0x7F).int()).to(torch.uint8).view(torch.float8_e4m3fn)

    copies = copies_for(M * K + N * K + 2 * M * N, 64)
    As = [codes(M, K) for _ in range(copies)]
    Bs = [codes(N, K) for _ in range(copies)]
    one = torch.ones((), device=dev)
    sa = torch.rand((M, 1), device=dev, generator=gen) + 0.5
    sb = torch.rand((1, N), device=dev, generator=gen) + 0.5
    stream = torch.cuda.Stream()
    lines = []
    for name, (x, y) in (("per tensor", (one, one)), ("per row of A and column of B", (sa, sb))):
        def step(i):
            torch._scaled_mm(As[i % copies], Bs[i % copies].t(), scale_a=x, scale_b=y, out_dtype=torch.bfloat16)

        try:
            ms, _ = time_steps(step, copies, steps, 5, False, stream, torch)
        except RuntimeError as e:   # the library may not offer a scaling mode
            lines.append({"floor": "library_fp8_gemm", "scales": name, "error": str(e)[:160]})
            continue
        us = ms / steps * 1e3
        lines.append({"floor": "library_fp8_gemm", "scales": name, "M": M, "N": N, "K": K, "us": round(us, 2),
                      "tflops": round(2 * M * N * K / us / 1e6, 1)})
    return lines


def copy_only(nbytes, torch, reps=5):
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 100 for the prefill shape, 4096 for the others)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default: 10 / 256)")
    ap.add_argument("--workload", default="prefill_16384x4096x4096")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the named workload (the headline line without per_config)")
    ap.add_argument("--out", default=None, help="output dtype (default: the workload's first)")
    ap.add_argument("--M", type=int, default=None, help="a sweep point of the workload")
    ap.add_argument("--N", type=int, default=None, help="another N for the workload's M and K (tuning)")
    ap.add_argument("--K", type=int, default=None, help="another K, a multiple of 128 (tuning)")
    ap.add_argument("--probe-load", default=None, help="the load-path probe, one JSON line per case to FILE")
    ap.add_argument("--max-copies", type=int, default=1024)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-library", action="store_true",
                    help="skip the platform library's FP8 GEMM reference on the MFMA-bound shape")
    ap.add_argument("--sweep", default=None)
    ap.add_argument("--dispatch-sweep", default=None,
                    help="time the dispatcher's choice against every forced alternative on the pages' shape sets")
    ap.add_argument("--floors", default=None, help="launch and streaming floors of the GPU, to FILE")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--variant", default="auto", help="force a kernel variant (tuning)")
    ap.add_argument("--split", type=int, default=0, help="force a split-K count (tuning)")
    ap.add_argument("--cfg", type=int, default=None, help="force a tile configuration (tuning)")
    ap.add_argument("--op", default="gemm", choices=["gemm", "quantize", "quantize_weights", "grouped"],
                    help="gemm (default), the activation quantiser on the workload's A shape, "
                         "the 128x128 weight quantiser on its B shape, or the grouped MoE GEMM")
    ap.add_argument("--moe", default="moe_decode_t64_e256_512x4096", help="MoE workload of --op grouped")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the library runs on one GPU; sharding the GEMM over several GPUs "
                                   "(by N, M or K) is a design note, not a measured path",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if args.copy_bytes:
        copy_only(args.copy_bytes, torch)
        return
    import block_scaled_fp8_gemm_amd as fbg
    import workloads as W
    fbg.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    if args.dispatch_sweep:
        dispatch_sweep(args.dispatch_sweep, torch, fbg)
        return
    if args.floors:
        platform_floors(args.floors, torch)
        return
    if args.probe_load:
        run_probe_load(args.probe_load, torch)
        return
    if args.sweep:
        with open(args.sweep, "w") as f:
            for name, w in W.WORKLOADS.items():
                for M in (w.M,) + tuple(m for m in w.sweep_M if m != w.M):
                    for out in w.out_dtypes:
                        steps = 200 if w.flops > 1e11 else 2048
                        r = run_workload(args, w, M, out, torch, fbg, W, steps, 20, not args.no_graph)
                        line = {"workload": name, "M": M, "N": w.N, "K": w.K, "out": out,
                                "variant": r["plan"]["variant_name"], "cfg": r["plan"]["config"],
                                "split_k": r["plan"]["split_k"], "grid": r["plan"]["grid"],
                                "us": round(r["ms_per_step"] * 1e3, 3), "tflops": round(r["tflops"], 2),
                                "gbs": round(r["gbs"], 1), "roofline": r["roof"], "copies": r["copies"],
                                "copy_floor_us": round(copy_floor_us(r["alg_bytes"], torch), 3)}
                        f.write(json.dumps(line) + "\n")
                        f.flush()
                        print(json.dumps(line), flush=True)
            for name, mw in W.MOE_WORKLOADS.items():   # the grouped (MoE) GEMM
                r = run_grouped(args, mw, torch, fbg, W, 400, 20, not args.no_graph)
                line = {"op": "grouped", "workload": name, "tokens": mw.tokens, "experts": mw.experts,
                        "top_k": mw.top_k, "rows": r["M"], "N": mw.N, "K": mw.K, "cfg": r["cfg"],
                        "active_experts": int((r["d"]["offsets"][1:] > r["d"]["offsets"][:-1]).sum()),
                        "us": round(r["ms_per_step"] * 1e3, 3), "tflops": round(r["tflops"], 2),
                        "gbs": round(r["gbs"], 1), "roofline": r["roof"], "copies": r["copies"]}
                f.write(json.dumps(line) + "\n")
                f.flush()
                print(json.dumps(line), flush=True)
            for name, w in W.WORKLOADS.items():     # the activation quantiser on each workload's A
                r = run_quantize(args, w, w.M, torch, fbg, 200 if w.M * w.K > 1e7 else 2048, 20, not args.no_graph)
                line = {"op": "quantize", "workload": name, "M": w.M, "K": w.K,
                        "us": round(r["ms_per_step"] * 1e3, 3), "gbs": round(r["gbs"], 1),
                        "roofline": r["roof"], "copies": r["copies"]}
                f.write(json.dumps(line) + "\n")
                f.flush()
                print(json.dumps(line), flush=True)
        return

    if args.op != "gemm":
        args.steps = args.steps if args.steps is not None else 400
        args.warmup = args.warmup if args.warmup is not None else 20
    if args.op == "grouped":
        mw = W.MOE_WORKLOADS[args.moe]
        out = args.out or "bf16"
        r = run_grouped(args, mw, torch, fbg, W, args.steps, args.warmup, not args.no_graph, out)
        line = {
            "metric": "HBM GB/s and % of roofline of the grouped (MoE) block-scaled FP8 GEMM, 1\u00d7MI355X",
            "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": mw.name, "tokens": mw.tokens, "experts": mw.experts, "top_k": mw.top_k,
                       "rows": r["M"], "N": mw.N, "K": mw.K, "out_dtype": out,
                       "active_experts": int((r["d"]["offsets"][1:] > r["d"]["offsets"][:-1]).sum()),
                       "tflops": round(r["tflops"], 3), "input_copies": r["copies"],
                       "graphs": not args.no_graph},
            "roofline": dict(r["roof"], traffic=None),
        }
        fl = copy_floor_us(r["alg_bytes"], torch)
        line["copy_floor"] = {"us": round(fl, 3), "bytes": r["alg_bytes"],
                              "frac_of_floor": round(fl / (r["ms_per_step"] * 1e3), 4)}
        rec = traffic_record(mw.name, out)
        if (rec is not None and args.cfg is None and rec.get("source_hash") == kernel_source_hash()
                and rec.get("variant") == "grouped" and rec.get("config") == r["cfg"] and rec.get("out") == out):
            line["roofline"]["traffic"] = rec["traffic_bytes"]
        line["config"]["cfg"] = r["cfg"]
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline_grouped(r["d"], r["flops"])
        print(json.dumps(line), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    M = args.M if args.M is not None else w.M
    reshaped = args.N is not None or args.K is not None
    if reshaped:
        # Another (N, K) for the workload's inputs recipe: named apart, so no
        # committed counter record (keyed by workload) applies to it.
        import dataclasses
        N_, K_ = args.N or w.N, args.K or w.K
        w = dataclasses.replace(w, name=f"{w.name}:N{N_}:K{K_}", N=N_, K=K_, sweep_M=())
    if args.op in ("quantize", "quantize_weights"):
        wts = args.op == "quantize_weights"
        r = run_quantize(args, w, M, torch, fbg, args.steps, args.warmup, not args.no_graph, weights=wts)
        M = r["rows"]
        line = {
            "metric": ("HBM GB/s and % of roofline of the 128x128 weight quantiser, 1\u00d7MI355X" if wts else
                       "HBM GB/s and % of roofline of the per-token 1x128 activation quantiser, 1\u00d7MI355X"),
            "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16->e4m3", "data": "synthetic",
            "config": {"workload": f"{'quantize_weights' if wts else 'quantize'}_{M}x{w.K}", "rows": M, "K": w.K,
                       "input_copies": r["copies"],
                       "graphs": not args.no_graph},
            "roofline": dict(r["roof"], traffic=None),
        }
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline_quantize(r["bits"], weights=wts)
        print(json.dumps(line), flush=True)
        return
    out = args.out or w.out_dtypes[0]
    steps = args.steps if args.steps is not None else (100 if w.flops > 1e11 else 4096)
    warmup = args.warmup if args.warmup is not None else (10 if w.flops > 1e11 else 256)
    r = run_workload(args, w, M, out, torch, fbg, W, steps, warmup, not args.no_graph,
                     args.variant, args.split, args.cfg)
    roof = dict(r["roof"])
    # The committed record is of the workload's own M (and N, K, by name).
    roof["traffic"] = profiled_traffic(w.name, r["plan"], out) if args.cfg is None and M == w.M else None
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "N": w.N, "K": w.K, "out_dtype": out,
                   "variant": r["plan"]["variant_name"], "tile": [r["plan"]["tile_m"], r["plan"]["tile_n"]],
                   "split_k": r["plan"]["split_k"], "grid": r["plan"]["grid"],
                   "input_copies": r["copies"], "graphs": not args.no_graph},
        "roofline": roof,
    }
    if args.cfg is not None:
        # The plan call reports the automatic tile; a forced configuration's
        # tile and grid are not known here.
        line["config"].update(forced_cfg=args.cfg, tile=None, grid=None)
    props = torch.cuda.get_device_properties(0)
    line["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                      "compute_units": props.multi_processor_count,
                      "memory_gib": round(props.total_memory / 2**30, 1)}
    fl = copy_floor_us(r["alg_bytes"], torch)
    line["copy_floor"] = {"us": round(fl, 3), "bytes": r["alg_bytes"],
                          "frac_of_floor": round(fl / (r["ms_per_step"] * 1e3), 4)}
    d = r.pop("d")
    r_us = r["ms_per_step"]
    del r
    if w.flops > 1e11 and not args.no_library and args.M is None and not reshaped:
        # The achievable reference of an MFMA-bound shape, on the same GPU in
        # the same run: the platform library's FP8 GEMM (no block scales).
        lib = library_fp8_gemm(torch, w.M, w.N, w.K)
        ref = {x["scales"]: x["us"] for x in lib if "us" in x}
        line["achievable"] = {"library_fp8_gemm_us": ref,
                              "frac_of_library": {k: round(v / (r_us * 1e3), 4) for k, v in ref.items()}}
    if not args.no_per_config and args.M is None and not reshaped and args.variant == "auto" and args.cfg is None:
        line["per_config"] = per_config(args, w.name, out, torch, fbg, W)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(line), flush=True)


# The other configurations of the metric (every (M,N,K) it is quoted on, and
# the prefill shape's second output dtype), each timed like the headline, plus
# the plain entry point fp8_block_gemm (no caller workspace) on the decode shape.
PER_CONFIG = [("small_16x512x256", "bf16", "ex"), ("decode_64x512x4096", "bf16", "ex"),
              ("decode_64x512x4096", "bf16", "fp8_block_gemm"), ("shortk_184x4096x256", "bf16", "ex"),
              ("midm_128x8192x1024", "bf16", "ex"), ("prefill_16384x4096x4096", "bf16", "ex"),
              ("prefill_16384x4096x4096", "fp32", "ex")]


def oracle_call_us(d, budget_s=1.0):
    """The oracle's time for one whole GEMM of a small workload on the
    host's cores (repeated for about `budget_s`)."""
    import oracle
    oracle.block_gemm(d["A"][:1], d["a_s"][:1], d["B"], d["b_s"])  # load the library
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            return el / reps * 1e6


def per_config(args, head_name, head_out, torch, fbg, W):
    """One entry per configuration of PER_CONFIG other than the headline's:
    us per call, TFLOP/s, roofline fraction, the fraction of a same-bytes
    device copy, and (small shapes) the oracle's time for the same GEMM on the
    host's cores.  Small shapes run 2000 steps over as many input copies (each
    copy read once after the MALL scrub), the prefill shape 20."""
    res = {}
    for name, out, entry in PER_CONFIG:
        if name == head_name and out == head_out and entry == "ex":
            continue
        w = W.WORKLOADS[name]
        big = w.flops > 1e11
        steps = 20 if big else 2000
        r = run_workload(args, w, w.M, out, torch, fbg, W, steps, 5 if big else 50, not args.no_graph,
                         entry=entry, max_copies=4 if big else 2048)
        fl = copy_floor_us(r["alg_bytes"], torch)
        key = f"{name}_{out}" + ("_fp8_block_gemm" if entry != "ex" else "")
        oracle_us = None
        if not big and not args.no_cpu and entry == "ex":
            oracle_us = oracle_call_us(r["d"])
        res[key] = {"M": w.M, "N": w.N, "K": w.K, "out_dtype": out, "entry": entry,
                    "variant": r["plan"]["variant_name"], "cfg": r["plan"]["config"],
                    "split_k": r["plan"]["split_k"], "grid": r["plan"]["grid"], "steps": steps,
                    "us": round(r["ms_per_step"] * 1e3, 3), "tflops": round(r["tflops"], 3),
                    "roofline": dict(r["roof"], traffic=profiled_traffic(name, r["plan"], out)),
                    "copy_floor_us": round(fl, 3),
                    "frac_of_floor": round(fl / (r["ms_per_step"] * 1e3), 4)}
        if oracle_us is not None:
            res[key]["oracle_us"] = round(oracle_us, 1)
            res[key]["gpu_speedup_over_oracle"] = round(oracle_us / (r["ms_per_step"] * 1e3), 1)
        print(f"per_config {key}: {res[key]['us']} us", file=sys.stderr, flush=True)
        del r
        torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
