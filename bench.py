"""Benchmark of the quantized linear layer on one MI355X.

Headline (the JSON line's `value`): the LLM.int8() mixed-precision linear at
the decode shape -- X fp16 [8 x 4096] with 6 outlier feature dims, W int8
[4096 x 4096] with per-channel fp32 scales, threshold 6.0, fp16 output.  One
step is one qa_qlinear_int8_mixed call (outlier detection, per-token int8
quantization, int8 MFMA GEMM, dequant epilogue, fp16 outlier product) on
inputs already resident in HBM.  Steps are replayed from a captured HIP graph
and cycle through copies of the weight so that every step reads it from HBM
rather than from the 256 MB Infinity Cache.  `value` is algorithmic bytes
moved per step / step time (GB/s).

Also reported (same JSON line, key "also"): whole-call throughput of the
prefill-shape mixed linear, the W8A8 FFN shape, the W4A4 group-Hadamard
linear, the SmoothQuant W8A8 linear on the prefill and FFN data and the
top-2% decomposition and the zero-point W8A8 linear on the prefill data, and
the Kronecker-transform W4A4 linear, the W4A8 group-Hadamard linear and the
W4A4 linear with zero-point activations (one-sided) on the W4A4 data, in int8
TOPS against the dense int8 MFMA peak; and the SmoothQuant and top-2% linears
at the decode shape (smooth_decode, topk_decode), in GB/s like the headline,
each with `gemv_roofline` from the recorded time of the fused decode kernel,
which is the whole call at this shape.  Each prefill-size entry carries
`gemm_roofline`:
the GEMM kernels' own time per call, the sum of their average rocprofv3
durations recorded in profiles/kernel_times.json for that workload (null while
the record is missing or any kernel source has changed since it was taken),
and the int8 TOPS and fraction of the dense peak that time gives.

roofline: the decode kernel's algorithmic bytes per launch / its average
launch duration, from HIP events recorded on the launch stream around the
timed region (every step is exactly one launch of that kernel).  `traffic` is
the HBM bytes per launch read from profiles/traffic.json (rocprofv3 FETCH_SIZE
and WRITE_SIZE of that kernel, each scaled by the same counter's reading for a
plain copy of known size, written by profile_counters.py), or null when that
record is missing or was taken on a different kernel source.
cpu_baseline: the CPU oracle timed on this host on whole decode steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantized-linear TOPS & % int8 MFMA peak; decode GB/s & % of 8 TB/s"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5033.2            # 256 CU x 2.4 GHz x 8192 int8 ops / clk / CU (dense)
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--no-also", action="store_true", help="skip the prefill / W8A8 / W4A4 / SmoothQuant lines")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--only", default=None,
                   help="run one workload only (decode|prefill|w8a8|w4a4|smooth_prefill|smooth_ffn|topk_prefill|"
                        "asym_prefill|kron_w4a4|w4a8|w4a4_asym|smooth_decode|topk_decode|copy|floor), for "
                        "profiling; copy is a plain "
                        "1 GiB device copy used to calibrate HBM byte counters; floor sweeps the plain "
                        "read of the decode step's bytes (qa_probe_stream_read) and an empty launch")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class GraphSteps:
    """Capture calls into HIP graphs: `run(k)` replays exactly k calls, taken
    in turn from `fns` (call i runs fns[i % len(fns)])."""

    def __init__(self, torch, fns):
        self.torch = torch
        self.fns = fns
        self.n = len(fns)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graphs = {}

    def graph(self, k):
        if k not in self.graphs:
            g = self.torch.cuda.CUDAGraph()
            with self.torch.cuda.graph(g):
                for i in range(k):
                    self.fns[i % self.n]()
            self.graphs[k] = g
        return self.graphs[k]


def time_graph(torch, gs, steps, warmup):
    """Replay `warmup` untimed calls, then time exactly `steps` calls (one graph
    holding that many) between HIP events on the replay stream; returns
    (ms per call, wall ms per call, calls timed)."""
    steps = max(1, int(steps))
    g = gs.graph(steps)
    if warmup > 0:
        gs.graph(int(warmup)).replay()
    g.replay()                              # first replay of a fresh graph uploads it: untimed
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return e0.elapsed_time(e1) / steps, wall / steps, steps


def recorded_traffic(kernel, source):
    """HBM bytes per launch of `kernel` from profiles/traffic.json, or None if
    there is no record or it was taken on a different version of `source`."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
        with open(os.path.join(ROOT, source), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source") != source or rec.get("source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def recorded_gemm_time(key, tag="k_gemm"):
    """GEMM-kernel time per call of workload `key` from profiles/kernel_times.json
    (rocprofv3 --kernel-trace of `bench.py --only key`, written by
    profile_counters.py): the sum of the average durations of its kernels
    whose names contain `tag` (k_gemm_*, or k_gemv_* at decode sizes), each
    of which runs once per call.  (None, reason) when the record
    is missing or any kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(path):
        return None, None, "no profiles/kernel_times.json"
    with open(path) as f:
        rec = json.load(f).get(key)
    if rec is None:
        return None, None, "no record for %s" % key
    csrc = os.path.join(ROOT, "bit_quantized_linear_int8_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            if rec["sources_sha256"].get(name) != hashlib.sha256(fh.read()).hexdigest():
                return None, None, "kernel sources changed since the record (%s)" % name
    gemm = {k: v for k, v in rec["kernels"].items() if tag in k}
    if not gemm or len({v["calls"] for v in gemm.values()}) != 1:
        return None, None, "record has no single set of GEMM launches"
    return sum(v["avg_us"] for v in gemm.values()), sorted(gemm), rec["command"]


# --------------------------------------------------------------------------- workloads
def decode_workload(torch, qa, synthetic, dev):
    c = synthetic.config("decode_mixed")
    M, K, N = c["M"], c["K"], c["N"]
    X = torch.from_numpy(c["X"]).to(dev)
    W16 = torch.from_numpy(c["W"]).to(dev)
    Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
    del W16
    copies = max(2, -(-2 * MALL_BYTES // (N * K)))
    Wqs = [Wq] + [Wq.clone() for _ in range(copies - 1)]
    sws = [s_w] + [s_w.clone() for _ in range(copies - 1)]
    out = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = torch.empty(qa.qa_qlinear_int8_mixed_workspace(M, K), dtype=torch.uint8, device=dev)

    def mk(i):
        return lambda: qa.qa_qlinear_int8_mixed(X, Wqs[i], sws[i], None, c["tau"], out=out, workspace=ws)
    fns = [mk(i) for i in range(copies)]
    # algorithmic bytes per call: int8 weight + fp32 channel scales + fp16 X read + fp16 out written
    nbytes = N * K + 4 * N + 2 * M * K + 2 * M * N
    return c, fns, nbytes, copies


def prefill_like(torch, qa, synthetic, dev, name):
    c = synthetic.config(name)
    M, K, N = c["M"], c["K"], c["N"]
    X = torch.from_numpy(c["X"]).to(dev)
    W16 = torch.from_numpy(c["W"]).to(dev)
    Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
    del W16
    odt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[c["out_dtype"]]
    out = torch.empty((M, N), dtype=odt, device=dev)
    ws = torch.empty(qa.qa_qlinear_int8_mixed_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_int8_mixed(X, Wq, s_w, None, c["tau"], out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def smooth_workload(torch, qa, synthetic, dev, name, per_tensor):
    """SmoothQuant W8A8 on a workload's data: device calibration (column maxima
    of X and W, alpha = 0.5 factors), offline smoothed weight, then the timed
    call (smoothing + int8 quantization of X, int8 GEMM, dequant)."""
    c = synthetic.config(name)
    M, K, N = c["M"], c["K"], c["N"]
    X = torch.from_numpy(c["X"]).to(dev)
    W16 = torch.from_numpy(c["W"]).to(dev)
    s = qa.qa_smooth_factors(qa.qa_col_absmax(X), qa.qa_col_absmax(W16), 0.5)
    Wq, s_w = qa.qa_quantize_smooth_int8(W16, s, multiply=True)
    del W16
    odt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[c["out_dtype"]]
    out = torch.empty((M, N), dtype=odt, device=dev)
    ws = torch.empty(qa.qa_qlinear_int8_smooth_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=per_tensor, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def topk_workload(torch, qa, synthetic, dev, name, share):
    """LLM.int8() with the top `share` of the K dimensions decomposed (instead
    of the threshold) on a workload's data."""
    c = synthetic.config(name)
    M, K, N = c["M"], c["K"], c["N"]
    X = torch.from_numpy(c["X"]).to(dev)
    Wq, s_w = qa.qa_quantize_rowwise_int8(torch.from_numpy(c["W"]).to(dev))
    k = qa.topk_count(share, K)
    odt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[c["out_dtype"]]
    out = torch.empty((M, N), dtype=odt, device=dev)
    ws = torch.empty(qa.qa_qlinear_int8_topk_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_int8_topk(X, Wq, s_w, k, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K, k


def decode_variant_workload(torch, qa, synthetic, dev, kind):
    """The SmoothQuant (per-token) or top-2% linear at the decode shape, over
    weight copies like the decode headline (every call streams its weight
    from HBM); -> (config, calls, algorithmic bytes per call, label)."""
    c = synthetic.config("decode_mixed")
    M, K, N = c["M"], c["K"], c["N"]
    X = torch.from_numpy(c["X"]).to(dev)
    W16 = torch.from_numpy(c["W"]).to(dev)
    out = torch.empty((M, N), dtype=torch.float16, device=dev)
    if kind == "smooth":
        s = qa.qa_smooth_factors(qa.qa_col_absmax(X), qa.qa_col_absmax(W16), 0.5)
        Wq, s_w = qa.qa_quantize_smooth_int8(W16, s, multiply=True)
        ws = torch.empty(qa.qa_qlinear_int8_smooth_workspace(M, K), dtype=torch.uint8, device=dev)
        call = lambda W: (lambda: qa.qa_qlinear_int8_smooth(X, s, W, s_w, out=out, workspace=ws))
        nbytes = N * K + 4 * N + 2 * M * K + 4 * K + 2 * M * N
        label = "smooth_decode: SmoothQuant W8A8 (X/s per-token int8), decode_mixed data"
    else:
        Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
        k = qa.topk_count(0.02, K)
        ws = torch.empty(qa.qa_qlinear_int8_topk_workspace(M, K), dtype=torch.uint8, device=dev)
        call = lambda W: (lambda: qa.qa_qlinear_int8_topk(X, W, s_w, k, out=out, workspace=ws))
        nbytes = N * K + 4 * N + 2 * M * K + 2 * M * N
        label = "topk_decode: LLM.int8() with the top 2%% (%d) of dims in fp16, decode_mixed data" % k
    del W16
    copies = max(2, -(-2 * MALL_BYTES // (N * K)))
    Wqs = [Wq] + [Wq.clone() for _ in range(copies - 1)]
    return c, [call(W) for W in Wqs], nbytes, label


def asym_workload(torch, qa, synthetic, dev, name):
    """W8A8 with per-token zero-point activations and a zero-point weight on a
    workload's data."""
    c = synthetic.config(name)
    M, K, N = c["M"], c["K"], c["N"]
    X = torch.from_numpy(c["X"]).to(dev)
    Wq, s_w, z_w, rw = qa.qa_quantize_rowwise_int8_asym(torch.from_numpy(c["W"]).to(dev))
    odt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[c["out_dtype"]]
    out = torch.empty((M, N), dtype=odt, device=dev)
    ws = torch.empty(qa.qa_qlinear_int8_asym_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_int8_asym(X, Wq, s_w, rw, z_w=z_w, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def kron_workload(torch, qa, synthetic, dev):
    """FlatQuant's apply stage on the W4A4 workload: 64 x 64 Kronecker factors
    (random orthogonal stand-ins), transform + int4 of X fused, W4A4 GEMM with
    the offline-transformed per-group int4 weight."""
    c = synthetic.config("w4a4_hadamard")
    M, K, N, G = c["M"], c["K"], c["N"], c["G"]
    n1, n2 = 64, K // 64
    P1, P2 = synthetic.kron_factors(n1, n2, seed=0)
    P1 = torch.from_numpy(P1).to(dev)
    P2 = torch.from_numpy(P2).to(dev)
    X = torch.from_numpy(c["X"]).to(dev)
    Wp, s_w = qa.qa_kron_quant_int4(torch.from_numpy(c["W"]).to(dev), P1, P2, G=G)   # orthogonal: P^-T = P
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(qa.qa_qlinear_kron_w4a4_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_kron_w4a4(X, P1, P2, Wp, s_w, G=G, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def w4a4_workload(torch, qa, synthetic, dev):
    c = synthetic.config("w4a4_hadamard")
    M, K, N, G = c["M"], c["K"], c["N"], c["G"]
    X = torch.from_numpy(c["X"]).to(dev)
    Wp, s_w = qa.qa_hadamard_quant_int4(torch.from_numpy(c["W"]).to(dev), G, True)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(qa.qa_qlinear_w4a4_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_w4a4(X, Wp, s_w, G=G, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def w4a4_asym_workload(torch, qa, synthetic, dev):
    """The W4A4 weight with zero-point int4 activations; the activations are
    made one-sided (|X|), the case the zero-point is for."""
    c = synthetic.config("w4a4_hadamard")
    M, K, N, G = c["M"], c["K"], c["N"], c["G"]
    import numpy as np
    X = torch.from_numpy(np.abs(c["X"])).to(dev)
    Wp, s_w = qa.qa_hadamard_quant_int4(torch.from_numpy(c["W"]).to(dev), G, True)
    c_w = qa.qa_w4_column_terms(Wp, s_w, K, G)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(qa.qa_qlinear_w4a4_asym_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_w4a4_asym(X, Wp, s_w, c_w, G=G, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def w4a8_workload(torch, qa, synthetic, dev):
    """The W4A4 data with 8-bit activations: group-Hadamard int8 codes of X
    against the same offline per-group int4 weight."""
    c = synthetic.config("w4a4_hadamard")
    M, K, N, G = c["M"], c["K"], c["N"], c["G"]
    X = torch.from_numpy(c["X"]).to(dev)
    Wp, s_w = qa.qa_hadamard_quant_int4(torch.from_numpy(c["W"]).to(dev), G, True)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(qa.qa_qlinear_w4a8_workspace(M, K), dtype=torch.uint8, device=dev)
    fns = [lambda: qa.qa_qlinear_w4a8(X, Wp, s_w, G=G, out=out, workspace=ws)]
    return c, fns, 2 * M * N * K


def read_floor(torch, qa, dev, steps, warmup):
    """The single-launch floor the decode kernel is measured against: one plain
    read of the decode step's bytes (16,924,672 B at 8 x 4096 x 4096) per
    launch, from as many buffer copies as the decode bench uses (every launch
    reads HBM), timed like the decode steps (HIP-graph replay, events around
    exactly `steps` launches), over workgroup counts, bytes per lane and
    load, and loads in flight per lane; and the same grid with nothing to
    read (the launch cost)."""
    M = K = N = 4096
    nbytes = N * K + 4 * N + 2 * 8 * K + 2 * 8 * N
    copies = max(2, -(-2 * MALL_BYTES // nbytes))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.empty(2048 * 512, dtype=torch.int32, device=dev)
    steps, warmup = min(int(steps), 256), min(int(warmup), 32)

    def run(nb, wgs, lb, u):
        fns = [(lambda b=b: qa.qa_probe_stream_read(b, nb, wgs, lb, u, sink=sink)) for b in bufs]
        ms, _, n = time_graph(torch, GraphSteps(torch, fns), steps, warmup)
        return ms * 1e3
    empty = run(0, 256, 16, 1)
    sweep = []
    for wgs in (256, 512, 1024, 2048):
        for lb in (16, 8, 4):
            for u in (1, 4, 8):
                us = run(nbytes, wgs, lb, u)
                sweep.append({"wgs": wgs, "lane_bytes": lb, "unroll": u, "us": round(us, 3),
                              "GBs": round(nbytes / (us * 1e-6) / 1e9, 1)})
                log("[floor] wgs %4d lane_bytes %2d unroll %d: %.3f us" % (wgs, lb, u, us))
    best = min(sweep, key=lambda r: r["us"])
    return {"bytes": nbytes, "copies": copies, "launches_timed": steps, "empty_launch_us": round(empty, 3),
            "best": best, "sweep": sweep}


# --------------------------------------------------------------------------- CPU oracle baseline
def cpu_baseline(c, nbytes, seconds):
    import numpy as np
    import oracle
    Wq, s_w = oracle.quant_rows(c["W"])
    s_w = s_w[:, 0]
    oracle.qlinear_int8_mixed(c["X"], Wq, s_w, tau=c["tau"])         # warm
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.qlinear_int8_mixed(c["X"], Wq, s_w, tau=c["tau"])
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole decode steps (all 8 tokens x 4096 channels) of the plain-C oracle, %.1f s, "
                      "%.1f ms per step" % (n, el, per * 1e3)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and has no multi-GPU "
              "path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_linear_int8_amd as qa
    import synthetic
    qa.lib()
    dev = torch.device("cuda:0")

    result = None
    also = []
    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        print(json.dumps({"copy_bytes": n, "ms": round(ms, 4), "read_write_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1)}))
        return
    if args.only == "floor":
        print(json.dumps({"floor": read_floor(torch, qa, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.only in (None, "decode"):
        log("[bench] decode_mixed: building inputs")
        c, fns, nbytes, copies = decode_workload(torch, qa, synthetic, dev)
        gs = GraphSteps(torch, fns)
        log("[bench] decode_mixed: timing %d steps (graph of %d)" % (args.steps, gs.n))
        ms, wall_ms, n = time_graph(torch, gs, args.steps, args.warmup)
        gbs = nbytes / (ms * 1e-3) / 1e9
        ach = gbs                       # one launch of the decode kernel per step
        result = {
            "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": n,
            "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "i8", "data": "synthetic",
            "config": {"workload": "decode_mixed: LLM.int8() mixed linear, X fp16 [8 x 4096] (6 outlier dims), "
                                   "W int8 [4096 x 4096] + fp32 channel scales, threshold 6.0, fp16 out",
                       "M": c["M"], "K": c["K"], "N": c["N"], "threshold": c["tau"], "weight_copies": copies,
                       "bytes_per_step": nbytes, "launch": "HIP graph replay", "wall_ms_per_step": round(wall_ms, 6)},
            "roofline": {"bound": "hbm", "kernel": "k_decode_mixed", "achieved": round(ach, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("k_decode_mixed",
                                                     "bit_quantized_linear_int8_amd/csrc/k_decode.hip"),
                         "kernel_ms_avg": round(ms, 6), "algorithmic_bytes": nbytes},
        }
        log("[bench] decode: %.1f GB/s, %.2f us per launch" % (gbs, ms * 1e3))
        if not args.no_cpu:
            log("[bench] cpu oracle baseline (~%.0f s)" % args.cpu_seconds)
            result["cpu_baseline"] = cpu_baseline(c, nbytes, args.cpu_seconds)
        del fns, gs
        torch.cuda.empty_cache()

    keys = ("prefill", "w8a8", "w4a4", "smooth_prefill", "smooth_ffn", "topk_prefill", "asym_prefill", "kron_w4a4",
            "w4a8", "w4a4_asym", "smooth_decode", "topk_decode")
    run_also = (args.only is None and not args.no_also) or args.only in keys
    if run_also:
        todo = []
        for name, key in (("prefill_mixed", "prefill"), ("w8a8_ffn", "w8a8"), ("w4a4_hadamard", "w4a4"),
                          ("prefill_mixed", "smooth_prefill"), ("w8a8_ffn", "smooth_ffn"),
                          ("prefill_mixed", "topk_prefill"), ("prefill_mixed", "asym_prefill"),
                          ("w4a4_hadamard", "kron_w4a4"), ("w4a4_hadamard", "w4a8"),
                          ("w4a4_hadamard", "w4a4_asym"), ("decode_mixed", "smooth_decode"),
                          ("decode_mixed", "topk_decode")):
            if args.only in (None, key):
                todo.append((name, key))
        for name, key in todo:
            log("[bench] %s: building inputs" % key)
            if key in ("smooth_decode", "topk_decode"):
                c, fns, nbytes, name = decode_variant_workload(torch, qa, synthetic, dev, key.split("_")[0])
                gs = GraphSteps(torch, fns)
                log("[bench] %s: timing %d calls" % (name, args.steps))
                ms, wall_ms, n = time_graph(torch, gs, args.steps, args.warmup)
                gbs = nbytes / (ms * 1e-3) / 1e9
                # both calls are one launch of the fused decode kernel at this shape
                gus, gnames, gsrc = recorded_gemm_time(key, "k_decode_mixed")
                if gus is None:
                    gemv = {"kernel_us": None, "reason": gsrc}
                else:
                    gemv = {"bound": "hbm", "kernels": gnames, "kernel_us": round(gus, 3),
                            "achieved": round(nbytes / (gus * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(nbytes / (gus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "source": "profiles/kernel_times.json[%s]: %s" % (key, gsrc)}
                also.append({"workload": name, "key": key, "M": c["M"], "K": c["K"], "N": c["N"],
                             "ms_per_call": round(ms, 6), "GBs": round(gbs, 2), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                             "bytes_per_call": nbytes, "calls": n,
                             "note": "whole call (all kernels), graph replay over weight copies",
                             "gemv_roofline": gemv})
                log("[bench] %s: %.2f us per call, %.1f GB/s" % (name, ms * 1e3, gbs))
                del fns, gs
                torch.cuda.empty_cache()
                continue
            if key == "w4a4":
                c, fns, ops = w4a4_workload(torch, qa, synthetic, dev)
            elif key == "smooth_prefill":
                c, fns, ops = smooth_workload(torch, qa, synthetic, dev, name, per_tensor=False)
                name = "smoothquant_prefill: X/s per-token int8, %s data" % name
            elif key == "topk_prefill":
                c, fns, ops, k = topk_workload(torch, qa, synthetic, dev, name, 0.02)
                name = "topk_prefill: LLM.int8() with the top 2%% (%d) of dims in fp16, %s data" % (k, name)
            elif key == "kron_w4a4":
                c, fns, ops = kron_workload(torch, qa, synthetic, dev)
                name = "kron_w4a4: FlatQuant Kronecker transform (64 x 64) + W4A4, %s data" % name
            elif key == "w4a4_asym":
                c, fns, ops = w4a4_asym_workload(torch, qa, synthetic, dev)
                name = "w4a4_asym: group-Hadamard W4A4, zero-point int4 activations, one-sided %s data" % name
            elif key == "w4a8":
                c, fns, ops = w4a8_workload(torch, qa, synthetic, dev)
                name = "w4a8: group-Hadamard int8 activations x per-group int4 weight, %s data" % name
            elif key == "asym_prefill":
                c, fns, ops = asym_workload(torch, qa, synthetic, dev, name)
                name = "asym_prefill: W8A8 with zero-point activations and weight, %s data" % name
            elif key == "smooth_ffn":
                c, fns, ops = smooth_workload(torch, qa, synthetic, dev, name, per_tensor=True)
                name = "smoothquant_ffn: X/s per-tensor int8, %s data" % name
            else:
                c, fns, ops = prefill_like(torch, qa, synthetic, dev, name)
            gs = GraphSteps(torch, fns)
            st = min(args.steps, 64)
            log("[bench] %s: timing %d calls" % (name, st))
            ms, wall_ms, n = time_graph(torch, gs, st, min(args.warmup, 8))
            tops = ops / (ms * 1e-3) / 1e12
            gus, gnames, gsrc = recorded_gemm_time(key)
            if gus is None:
                gemm = {"kernel_us": None, "reason": gsrc}
            else:
                gt = ops / (gus * 1e-6) / 1e12
                gemm = {"bound": "mfma", "kernels": gnames, "kernel_us": round(gus, 3), "achieved": round(gt, 2),
                        "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gt / INT8_PEAK_TOPS, 4),
                        "weights": "warm (one weight, re-read every call)",
                        "source": "profiles/kernel_times.json[%s]: %s" % (key, gsrc)}
            also.append({"workload": name, "key": key, "M": c["M"], "K": c["K"], "N": c["N"],
                         "ms_per_call": round(ms, 5), "int8_tops": round(tops, 2),
                         "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4), "calls": n,
                         "note": "whole call (all kernels), graph replay, weights warm", "gemm_roofline": gemm})
            log("[bench] %s: %.3f ms per call, %.1f TOPS" % (name, ms, tops))
            del fns, gs
            torch.cuda.empty_cache()

    if result is None:
        print(json.dumps({"also": also}))
        return
    result["also"] = also
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
