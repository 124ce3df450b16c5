#!/usr/bin/env python3
"""Benchmark of the DSA decode hot path on one MI355X.

Workload (one "step"): one fused DSA decode step -- lightning-indexer scan of
a 1,048,576-token history (+1 new token), top-2,048 selection and sparse GQA-4
attention with sink -- for batch 1, one query token (dsa_decode_1m).  Inputs
are seeded synthetic tensors resident in HBM before the timed region; R = 4
instances of every input rotate so the 256 MB Infinity Cache cannot serve the
134 MB key stream from one step to the next.

Printed (one JSON line):
  value     whole-step HBM throughput = algorithmic bytes / step time (GB/s)
  roofline  the step's dominant kernel, its index scan (idx_scan_kernel<1,
            true>, which also leaves each workgroup's top-32 list): the scan
            kernel nodes are taken out of a captured step and replayed alone,
            timed with HIP events on their launch stream; algorithmic bytes
            per launch (keys, index query, weights) / mean launch time,
            against the 8 TB/s HBM peak and against a streaming-read ceiling
            measured in the same run
  prefill_indexer  the fp8 MFMA contraction of an 8,192-token prefill chunk
            against 1,056,768 keys (causal): achieved TFLOP/s and % of the
            5.0 PFLOP/s dense fp8 peak
  cache_append     the step that appends new tokens to the caches (LayerNorm,
            partial RoPE, fp8/bf16 rounding, cache writes): one decode token,
            and a full 8,192-token prefill chunk as HBM GB/s
  small_decode     the 8K-key decode step and the 4-token verify at 128K
            (latency per step; their caches stay in the Infinity Cache)
  cpu_baseline     the fp64 oracle's decode step on this host, on a bounded
            sample, in the same unit
"""
import argparse
import json
import os
import sys
import time

# the CPU baseline's BLAS / OpenMP threads: every core this process may run on,
# fixed before numpy is first imported (an existing setting is kept)
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(len(os.sched_getaffinity(0))))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
ROTATE = 4

# algorithmic bytes of one dsa_decode_1m step
L, T, K = 1048576, 1, 2048
K_TOP = K
LK = L + T
BYTES_KEYS = LK * 128
BYTES_GATHER = K * 4 * (192 + 128) * 2
BYTES_SMALL = T * 64 * 192 * 2 + T * 64 * 128 * 2 + T * 16 * 128 + T * 16 * 4 + 64 * 4
STEP_BYTES = BYTES_KEYS + BYTES_GATHER + BYTES_SMALL            # 139,504,064
SCAN_BYTES = BYTES_KEYS + T * 16 * 128 + T * 16 * 4 + T * LK * 4  # standalone scan: keys + q + w + scores out
LIST_SCAN_BYTES = BYTES_KEYS + T * 16 * 128 + T * 16 * 4         # the step's scan: keys + q + w (134,219,968)

PREFILL_T, PREFILL_L = 8192, 1048576
PREFILL_LK = PREFILL_L + PREFILL_T


def prefill_flops():
    # causal visible (t, s) pairs x 16 heads x 128 dims x 2
    pairs = PREFILL_T * (PREFILL_LK - PREFILL_T) + PREFILL_T * (PREFILL_T + 1) // 2
    return pairs * 16 * 128 * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-batch", action="store_true")
    ap.add_argument("--no-recall", action="store_true")
    ap.add_argument("--no-swa", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=10)
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="also run 4 plain device copies of this many bytes (calibrates HBM counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported"}))
        sys.exit(2)
    import numpy as np
    import torch

    from sparse_long_context_index_amd import binding, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    binding.load()
    if args.copy_calib:
        src = torch.empty(args.copy_calib, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = synth.CONFIGS["dsa_decode_1m"]
    t0 = time.time()
    d = synth.decode_inputs(cfg)
    gen_s = time.time() - t0

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    base = {n: up(d[n]) for n in ("q_idx", "w", "k_idx", "q", "k", "v", "sink")}
    inst = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(ROTATE - 1)]
    sm = float(d["sm_scale"])
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_DECODE_STEP, LK, T, K))
    outs = [torch.empty((T, 64, 128), dtype=torch.bfloat16, device=dev) for _ in range(ROTATE)]
    st = torch.cuda.current_stream()

    def step(i):
        x = inst[i % ROTATE]
        binding.dsa_decode_step(x["q_idx"], x["w"], x["k_idx"], x["q"], x["k"], x["v"], LK, T, K,
                                x["sink"], sm, out=outs[i % ROTATE], ws=ws)

    # one decode step per rotation instance, captured once and replayed (a
    # serving loop replays the step the same way; the launches then cost no
    # host time)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    g_step = capture(torch, lambda: [step(i) for i in range(ROTATE)])
    reps = max(1, -(-args.steps // ROTATE))
    n_steps = reps * ROTATE
    ms_replay, wall_ms = replay_ms(torch, g_step, reps)
    ms_step = ms_replay / ROTATE

    # the step's dominant kernel: its index scan, replayed alone (kernel nodes
    # taken from a captured step)
    try:
        ms_list_scan = time_step_scan(torch, step, reps)
        scan_err = None
    except (RuntimeError, OSError) as e:              # reported, and the standalone scan stands in
        ms_list_scan, scan_err = None, str(e)

    # the standalone scan (dsa_index_scores, which also stores the scores)
    scores = [torch.empty((T, LK), dtype=torch.float32, device=dev) for _ in range(ROTATE)]

    def scan(i):
        x = inst[i % ROTATE]
        binding.dsa_index_scores(x["q_idx"], x["w"], x["k_idx"], LK, T, scores=scores[i % ROTATE])

    for i in range(args.warmup):
        scan(i)
    torch.cuda.synchronize()
    # 4 rounds of the rotation per graph, so that the graph launch is spread
    # over 16 scans
    g_scan = capture(torch, lambda: [scan(i) for i in range(4 * ROTATE)])
    ms_scan = replay_ms(torch, g_scan, reps)[0] / (4 * ROTATE)
    scan_gbs = SCAN_BYTES / (ms_scan * 1e-3) / 1e9
    # the best streaming rate seen in this run: torch's own sum and copy over
    # 1 GiB, and this library's standalone scan (a read stream of the keys)
    ceiling = read_ceiling(torch, dev)
    ceiling["all"]["standalone scan"] = round(scan_gbs, 1)
    if scan_gbs > ceiling["GB/s"]:
        ceiling["GB/s"], ceiling["kernel"] = round(scan_gbs, 1), "idx_scan_kernel<1, false> (standalone scan)"
    if ms_list_scan is not None:
        rl_kernel, rl_bytes, rl_ms = "idx_scan_kernel<1, true> (the decode step's index scan)", LIST_SCAN_BYTES, ms_list_scan
    else:
        rl_kernel, rl_bytes, rl_ms = "idx_scan_kernel<1, false> (dsa_index_scores; step scan untimed: " + scan_err + ")", \
            SCAN_BYTES, ms_scan
    rl_gbs = rl_bytes / (rl_ms * 1e-3) / 1e9

    result = {
        "metric": "DSA decode-step µs & HBM GB/s (% peak) at 1M ctx; prefill indexer fp8 MFMA %",
        "value": round(STEP_BYTES / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "us_per_step": round(ms_step * 1e3, 3),
        "hbm_frac_of_peak": round(STEP_BYTES / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-index/bf16-attn/f32-acc",
        "data": "synthetic",
        "config": {"workload": "dsa_decode_1m", "history": L, "query_tokens": T, "topk": K,
                   "idx_heads": 16, "q_heads": 64, "kv_heads": 4, "qk_dim": 192, "v_dim": 128,
                   "algorithmic_bytes_per_step": STEP_BYTES, "rotation_instances": ROTATE},
        "roofline": {"bound": "hbm", "kernel": rl_kernel,
                     "achieved": round(rl_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(rl_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if ms_list_scan is not None else None,
                     "bytes_per_launch": rl_bytes, "us_per_launch": round(rl_ms * 1e3, 3),
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": round(rl_gbs / ceiling["GB/s"], 4),
                     "standalone_scan": {"kernel": "idx_scan_kernel<1, false> (dsa_index_scores, scores stored)",
                                         "bytes_per_launch": SCAN_BYTES, "us_per_launch": round(ms_scan * 1e3, 3),
                                         "achieved": round(scan_gbs, 2),
                                         "frac": round(scan_gbs / HBM_PEAK_GBS, 4)}},
        "host_wall_ms_per_step": round(wall_ms / n_steps, 6),
        "launch": "hip graph of one step per rotation instance, replayed",
        "input_gen_s": round(gen_s, 2),
    }

    if not args.no_append:
        result["cache_append"] = bench_append(torch, binding, dev, inst[0], reps)
    if not args.no_batch:
        result["decode_batch"] = bench_batch(torch, np, binding, synth, dev, reps)
    if not args.no_recall:
        result["index_recall"] = bench_recall(torch, binding, dev, inst[0], sm, reps)
    if not args.no_swa:
        result["swa_decode"] = bench_swa(torch, np, binding, synth, dev, reps)
    if not args.no_small:
        result["small_decode"] = bench_small(torch, np, binding, synth, dev, reps)
    if not args.no_prefill:
        del scores
        result["prefill_indexer"] = bench_prefill(torch, np, binding, synth, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, args.cpu_sample_steps)
    print(json.dumps(result), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "idx_scan_dsa_decode_1m_traffic.json")


def measured_traffic():
    """HBM bytes per launch of the step's scan from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (copy-calibrated), or None when the scan's
    sources have changed since those counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = hashlib.sha256()
        for p in rec["sources"]:
            h.update(open(os.path.join(ROOT, p), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["in_step_list_scan"]["traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def time_step_scan(torch, step, reps):
    """Mean launch time (ms) of the decode step's scan kernel alone.  One step
    per rotation instance is captured on a side stream (HIP stream capture
    through the runtime torch already loaded); the scan kernel nodes -- the
    grid of 512 x 256-thread workgroups -- are copied, with their captured
    arguments, into a graph that chains them 4 times over, and that graph is
    replayed between HIP events on the same stream."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")          # the runtime torch loaded

    class Dim3(ctypes.Structure):
        _fields_ = [("x", ctypes.c_uint), ("y", ctypes.c_uint), ("z", ctypes.c_uint)]

    class KernelNodeParams(ctypes.Structure):      # hipKernelNodeParams
        _fields_ = [("blockDim", Dim3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p),
                    ("gridDim", Dim3), ("kernelParams", ctypes.c_void_p), ("sharedMemBytes", ctypes.c_uint)]

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = ctypes.c_void_p()
    with torch.cuda.stream(side):
        ok(hip.hipStreamBeginCapture(ctypes.c_void_p(side.cuda_stream), 0), "hipStreamBeginCapture")
        for i in range(ROTATE):
            step(i)
        ok(hip.hipStreamEndCapture(ctypes.c_void_p(side.cuda_stream), ctypes.byref(graph)), "hipStreamEndCapture")
    n = ctypes.c_size_t(0)
    ok(hip.hipGraphGetNodes(graph, None, ctypes.byref(n)), "hipGraphGetNodes")
    nodes = (ctypes.c_void_p * n.value)()
    ok(hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)), "hipGraphGetNodes")
    scans = []
    for node in nodes:
        ty = ctypes.c_int(-1)
        ok(hip.hipGraphNodeGetType(ctypes.c_void_p(node), ctypes.byref(ty)), "hipGraphNodeGetType")
        if ty.value != 0:                          # hipGraphNodeTypeKernel
            continue
        p = KernelNodeParams()
        ok(hip.hipGraphKernelNodeGetParams(ctypes.c_void_p(node), ctypes.byref(p)), "hipGraphKernelNodeGetParams")
        # the grid may be recorded in workgroups or in threads
        if (p.gridDim.x in (512, 512 * 256) and (p.gridDim.y, p.gridDim.z) == (1, 1)
                and (p.blockDim.x, p.blockDim.y, p.blockDim.z) == (256, 1, 1)):
            scans.append(p)
    if len(scans) != ROTATE:
        raise RuntimeError(f"expected {ROTATE} scan kernel nodes, found {len(scans)}")
    g2 = ctypes.c_void_p()
    ok(hip.hipGraphCreate(ctypes.byref(g2), 0), "hipGraphCreate")
    prev = None
    for _ in range(4):
        for p in scans:
            node = ctypes.c_void_p()
            deps = (ctypes.c_void_p * 1)(prev) if prev is not None else None
            ok(hip.hipGraphAddKernelNode(ctypes.byref(node), g2, deps, 1 if prev is not None else 0, ctypes.byref(p)),
               "hipGraphAddKernelNode")
            prev = node.value
    exe = ctypes.c_void_p()
    ok(hip.hipGraphInstantiate(ctypes.byref(exe), g2, None, None, 0), "hipGraphInstantiate")
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    for _ in range(3):
        ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * 4 * ROTATE)
    hip.hipGraphExecDestroy(exe)
    hip.hipGraphDestroy(g2)
    hip.hipGraphDestroy(graph)
    return ms


def read_ceiling(torch, dev, nbytes=1 << 30):
    """The streaming rates torch's own kernels reach over 1 GiB in this run:
    a float32 sum (reads N bytes) and a device copy (reads and writes N,
    counted as 2 N), each the best of 5 timed runs.  A reference point for
    what a plain stream achieves on this machine, not a bound of the kernels."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    y = torch.empty_like(x)
    out = {}
    for name, fn, moved in (("sum", lambda: x.sum(), nbytes), ("copy", lambda: y.copy_(x), 2 * nbytes)):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None or ms < best else best
        out[name] = round(moved / (best * 1e-3) / 1e9, 1)
    del x, y
    k = max(out, key=out.get)
    return {"GB/s": out[k], "kernel": f"torch {k} over 1 GiB", "all": out}


def capture(torch, fn):
    """Capture fn's launches (on torch's current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_ms(torch, g, reps):
    """Mean GPU ms per replay over `reps` back-to-back replays (HIP events on
    the replay stream) and the total host wall ms around them."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps, (time.perf_counter() - w0) * 1e3


def bench_prefill(torch, np, binding, synth, dev, chunk=1024, reps=2):
    """fp8 MFMA contraction of a full 8,192-token prefill chunk (row chunks of
    `chunk` tokens, scores materialised per chunk)."""
    rng = np.random.default_rng(11)
    q_idx = synth.encode_e4m3(rng.standard_normal((PREFILL_T, 16, 128)).astype(np.float32))
    w = rng.standard_normal((PREFILL_T, 16)).astype(np.float32)
    k_idx = synth.encode_e4m3(rng.standard_normal((PREFILL_LK, 128)).astype(np.float32))
    qd, wd, kd = (torch.from_numpy(a).to(dev) for a in (q_idx, w, k_idx))
    scores = torch.empty((chunk, PREFILL_LK), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream()

    def one_pass():
        for r0 in range(0, PREFILL_T, chunk):
            r1 = min(PREFILL_T, r0 + chunk)
            lk = PREFILL_LK - (PREFILL_T - r1)          # keys visible to the chunk's last row
            binding.dsa_index_scores(qd[r0:r1], wd[r0:r1], kd, lk, r1 - r0, scores=scores, ld=PREFILL_LK)

    one_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        one_pass()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = prefill_flops() / (ms * 1e-3) / 1e12
    res = {"workload": "dsa_prefill_1m_t8k indexer", "ms": round(ms, 3), "flops": prefill_flops(),
           "achieved": round(tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "bound": "mfma",
           "score_bytes_written": PREFILL_T * PREFILL_LK * 4}
    del scores
    # the fused index scores + top-2,048 of every row (no score matrix; the
    # selection on exact scores), timed with HIP events
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_PREFILL_TOPK, PREFILL_LK, PREFILL_T, 2048))
    idx = torch.empty((PREFILL_T, 2048), dtype=torch.int32, device=dev)
    binding.dsa_prefill_topk(qd, wd, kd, PREFILL_LK, PREFILL_T, 2048, idx=idx, ws=ws)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        binding.dsa_prefill_topk(qd, wd, kd, PREFILL_LK, PREFILL_T, 2048, idx=idx, ws=ws)
    e1.record(st)
    torch.cuda.synchronize()
    ms_f = e0.elapsed_time(e1) / reps
    tf_f = prefill_flops() / (ms_f * 1e-3) / 1e12
    res["fused_topk"] = {"workload": "dsa_prefill_1m_t8k index scores + top-2048 per row (fused)",
                         "ms": round(ms_f, 3), "achieved": round(tf_f, 1), "unit": "TFLOP/s",
                         "frac": round(tf_f / FP8_PEAK_TFLOPS, 4)}
    return res


# algorithmic bytes of the append step per new token: bf16 inputs (16 index
# query heads x 128, the index key, 64 query heads x 192, 4 KV heads x (192 +
# 128)) read once; fp8 index queries and key, bf16 queries, keys and values
# written once
APPEND_READ = 16 * 128 * 2 + 128 * 2 + 64 * 192 * 2 + 4 * 192 * 2 + 4 * 128 * 2
APPEND_WRITE = 16 * 128 + 128 + 64 * 192 * 2 + 4 * 192 * 2 + 4 * 128 * 2
APPEND_BYTES_PER_TOKEN = APPEND_READ + APPEND_WRITE               # 60,800


def bench_append(torch, binding, dev, x, reps):
    """dsa_cache_append: one decode token appended to the 1M-token caches
    (latency), and a full 8,192-token prefill chunk appended at positions
    1,048,576 .. 1,056,767 (HBM throughput).  Inputs are seeded N(0,1) bf16."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)

    def acts(T):
        r = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        return {"idx_q": r(T, 16, 128), "idx_k": r(T, 128), "q": r(T, 64, 192), "k": r(T, 4, 192),
                "v": r(T, 4, 128), "ln_gamma": 1 + 0.1 * torch.randn(128, generator=gen, device=dev),
                "ln_beta": 0.1 * torch.randn(128, generator=gen, device=dev)}

    def runner(a, T, Lk, kic, kc, vc):
        qi = torch.empty((T, 16, 128), dtype=torch.uint8, device=dev)
        qo = torch.empty((T, 64, 192), dtype=torch.bfloat16, device=dev)
        return lambda: binding.dsa_cache_append(a["idx_q"], a["idx_k"], a["q"], a["k"], a["v"], Lk, T, kic, kc, vc,
                                                ln_gamma=a["ln_gamma"], ln_beta=a["ln_beta"], q_idx_out=qi,
                                                q_out=qo)

    # decode: one token at position LK - 1 of the resident 1M caches
    one = runner(acts(1), 1, LK, x["k_idx"], x["k"].view(torch.bfloat16), x["v"].view(torch.bfloat16))
    one()
    torch.cuda.synchronize()
    g1 = capture(torch, lambda: [one() for _ in range(16)])
    us_one = replay_ms(torch, g1, max(reps, 10))[0] / 16 * 1e3

    # prefill chunk: 8,192 tokens
    T = PREFILL_T
    Lk = PREFILL_LK
    kic = torch.zeros((Lk, 128), dtype=torch.uint8, device=dev)
    kc = torch.zeros((Lk, 4, 192), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((Lk, 4, 128), dtype=torch.bfloat16, device=dev)
    big = runner(acts(T), T, Lk, kic, kc, vc)
    big()
    torch.cuda.synchronize()
    g8 = capture(torch, lambda: [big() for _ in range(4)])
    us_big = replay_ms(torch, g8, max(reps // 4, 10))[0] / 4 * 1e3
    nbytes = T * APPEND_BYTES_PER_TOKEN
    gbs = nbytes / (us_big * 1e-6) / 1e9
    del kic, kc, vc
    return {"kernel": "cache_append_kernel", "decode_t1_us": round(us_one, 3),
            "prefill": {"workload": "dsa_prefill_1m_t8k append", "tokens": T, "us": round(us_big, 3),
                        "bytes": nbytes, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"},
            "bytes_per_token": APPEND_BYTES_PER_TOKEN}


def decode_step_bytes(Lk, T, k):
    """Algorithmic bytes of one decode step: every visible index key, the
    gathered K/V of each token's k keys, queries, outputs, index queries,
    weights and the sink."""
    return (Lk * 128 + T * k * 4 * (192 + 128) * 2 + T * (64 * 192 * 2 + 64 * 128 * 2 + 16 * 128 + 16 * 4)
            + 64 * 4)


def bench_small(torch, np, binding, synth, dev, reps):
    """The two smaller decode workloads (8K-key history, one token; the
    4-token verify at 128K), one step per graph launch replayed.  Their index
    caches (1 MB, 16 MB) stay in the 256 MB Infinity Cache between replays,
    so the rates are latency figures, not HBM bandwidth."""
    out = {}
    for name in ("dsa_decode_8k", "dsa_verify_128k_t4"):
        cfg = synth.CONFIGS[name]
        d = synth.decode_inputs(cfg)
        x = {}
        for n in ("q_idx", "w", "k_idx", "q", "k", "v", "sink"):
            a = np.ascontiguousarray(d[n])
            x[n] = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        ws = binding.Workspace(binding.workspace_bytes(binding.OP_DECODE_STEP, cfg.Lk, cfg.T, cfg.k))
        o = torch.empty((cfg.T, 64, 128), dtype=torch.bfloat16, device=dev)
        sm = float(d["sm_scale"])

        def f():
            binding.dsa_decode_step(x["q_idx"], x["w"], x["k_idx"], x["q"], x["k"], x["v"], cfg.Lk, cfg.T, cfg.k,
                                    x["sink"], sm, out=o, ws=ws)
        for _ in range(5):
            f()
        torch.cuda.synchronize()
        g = capture(torch, lambda: [f() for _ in range(8)])
        ms = replay_ms(torch, g, max(reps // 8, 10))[0] / 8
        nbytes = decode_step_bytes(cfg.Lk, cfg.T, cfg.k)
        out[name] = {"history": cfg.L, "query_tokens": cfg.T, "topk": cfg.k, "us": round(ms * 1e3, 3),
                     "bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2)}
        del x, ws, o
    return out


def bench_batch(torch, np, binding, synth, dev, reps, B=64):
    """dsa_decode_batch: 64 sequences with key counts uniform in [256, 65536]
    (one new token each) sharing one cache; seeded N(0,1) inputs drawn on the
    device.  Algorithmic bytes: every sequence's index keys, the gathered K/V
    of its min(k, keys) selected rows, and its query, output and weights."""
    lens = synth.batch_lengths(B, 256, 65536, seed=1005)
    n_rows = int(lens.sum())
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    f8 = lambda *sh: torch.randn(sh, generator=gen, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
    bf = lambda *sh: torch.randn(sh, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    k_idx, K, V = f8(n_rows, 128), bf(n_rows, 4, 192), bf(n_rows, 4, 128)
    q_idx, q = f8(B, 1, 16, 128), bf(B, 1, 64, 192)
    w = torch.randn((B, 1, 16), generator=gen, device=dev)
    sink = torch.randn((64,), generator=gen, device=dev)
    st = torch.from_numpy(starts).to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    max_len = int(lens.max())
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_DECODE_BATCH, max_len, 1, K_TOP, B))
    out = torch.empty((B, 1, 64, 128), dtype=torch.bfloat16, device=dev)
    call = lambda: binding.dsa_decode_batch(q_idx, w, k_idx, q, K, V, st, sl, max_len, K_TOP, sink,
                                            1.0 / 192 ** 0.5, out=out, ws=ws)
    call()
    torch.cuda.synchronize()
    g = capture(torch, lambda: [call() for _ in range(4)])
    us = replay_ms(torch, g, max(reps // 4, 10))[0] / 4 * 1e3
    nbytes = int((lens * 128).sum() + (np.minimum(lens, K_TOP) * 4 * 320 * 2).sum()) + B * (2048 + 64 + 24576 + 16384)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "dsa_decode_batch b64 lengths U[256,65536] T=1 k=2048", "us": round(us, 3),
            "tokens_per_s": round(B / (us * 1e-6), 1), "bytes": nbytes, "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"}


def bench_recall(torch, binding, dev, x, sm, reps):
    """dsa_index_recall of the decode step's own top-2,048 at 1M keys: the
    dense pass reads every visible key's K row of all 4 KV heads."""
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    binding.dsa_decode_step(x["q_idx"], x["w"], x["k_idx"], x["q"], x["k"], x["v"], LK, T, K, x["sink"], sm,
                            idx_out=idx)
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_INDEX_RECALL, LK, T, K))
    rec = torch.empty((T, 64), dtype=torch.float32, device=dev)
    call = lambda: binding.dsa_index_recall(x["q"], x["k"], x["v"], LK, idx, sm, recall=rec, ws=ws)
    call()
    torch.cuda.synchronize()
    g = capture(torch, lambda: [call() for _ in range(4)])
    us = replay_ms(torch, g, max(reps // 4, 5))[0] / 4 * 1e3
    nbytes = LK * 4 * 192 * 2 + BYTES_GATHER + T * 64 * 192 * 2 + T * K * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "dsa_index_recall 1M keys, T=1, the decode step's top-2048", "us": round(us, 3),
            "bytes": nbytes, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
            "mean_recall": round(float(rec.mean().item()), 6)}


def bench_swa(torch, np, binding, synth, dev, reps):
    """swa_attn on the swa_decode_b64 workload: 64 sequences with lengths
    uniform in [256, 65536], one query token each, window 128, 8 KV heads;
    full-length ragged caches drawn on the device (only the windows are read).
    Algorithmic bytes: each sequence's window of K and V rows for 8 KV heads
    plus its query and output.  The graph replays 8 calls, one per instance:
    instance r has its own queries and outputs and shifts every sequence's
    start by 128 r rows (same lengths), so the 8 instances read disjoint
    windows -- 336 MB in all, more than the 256 MB Infinity Cache holds --
    and each call's windows come from HBM, not from the previous replay."""
    R = 8
    cfg = synth.CONFIGS["swa_decode_b64"]
    lens = synth._rng(cfg.seed, "seq_len").integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.B).astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    n_rows = int(lens.sum()) + (R - 1) * cfg.window
    gen = torch.Generator(device=dev)
    gen.manual_seed(51)

    def bf(*sh):
        t = torch.empty(sh, dtype=torch.bfloat16, device=dev)
        flat = t.view(-1)
        step = 1 << 28
        for i in range(0, flat.numel(), step):                 # float32 draws in 1 GiB pieces
            n = min(step, flat.numel() - i)
            flat[i:i + n] = torch.randn((n,), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        return t

    Kc, Vc = bf(n_rows, 8, 192), bf(n_rows, 8, 128)
    qs = [bf(cfg.B, 64, 192) for _ in range(R)]
    sink = torch.randn((64,), generator=gen, device=dev)
    sts = [torch.from_numpy(starts + cfg.window * r).to(dev) for r in range(R)]
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_SWA_ATTN, B=cfg.B))
    outs = [torch.empty((cfg.B, 64, 128), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    call = lambda r: binding.swa_attn(qs[r], Kc, Vc, sts[r], sl, cfg.window, sink, 1.0 / 192 ** 0.5, out=outs[r],
                                      ws=ws)
    call(0)
    torch.cuda.synchronize()
    g = capture(torch, lambda: [call(r) for r in range(R)])
    us = replay_ms(torch, g, max(reps // R, 10))[0] / R * 1e3
    nbytes = int(np.minimum(lens, cfg.window).sum()) * 8 * 320 * 2 + cfg.B * (64 * 192 * 2 + 64 * 128 * 2)
    gbs = nbytes / (us * 1e-6) / 1e9
    del Kc, Vc
    return {"workload": "swa_decode_b64 (64 sequences, window 128, GQA8)", "us": round(us, 3), "bytes": nbytes,
            "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "bound": "hbm (latency at this size)",
            "launch": f"graph of {R} calls over {R} instances with disjoint windows (reads from HBM)"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(d, n_steps):
    """The fp64 oracle's full decode step on a bounded sample of steps.  Its
    BLAS threads were fixed before numpy's import (module top); `cores` is
    the thread count the BLAS reports using."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    import oracle
    t0 = time.perf_counter()
    for _ in range(n_steps):
        oracle.dsa_decode_step(d, K)
    per = (time.perf_counter() - t0) / n_steps
    return {"value": round(STEP_BYTES / per / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "s_per_step": round(per, 3), "cpu_model": cpu_model(),
            "cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n_steps} full dsa_decode_1m steps (fp64 numpy oracle, same inputs)"}


if __name__ == "__main__":
    main()
