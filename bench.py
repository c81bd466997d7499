"""Benchmark of the packed ARCHead LM-head forward on one MI355X.

One step = one full forward of the packed head (projection, vocabulary-tile
kernel, top-1 reduction) over one batch of M synthetic bf16 hidden states,
with the packed fields already resident in HBM.  Steps are timed three
ways: launched one after another with HIP events around each step's
vocabulary-tile kernel (which gives the kernel time), launched back to back
with no events between them, and replayed from one HIP graph that holds 12
consecutive steps (as a decode loop captured in a graph runs them).  The
faster of the last two is the step time; all three are reported.  The headline workload is the
Qwen3-8B-shaped head (V=151936, d=4096, k=256, r=64, g=128) at M=1 (decode).
Three independent copies of the packed head are rotated so that no step finds
the previous step's 357 MB in the 256 MB last-level cache.

Prints ONE JSON line.  Besides the headline numbers it carries:
  roofline      the vocabulary-tile kernel against HBM bandwidth; its time is
                taken with HIP events recorded by the library on the same
                stream immediately around that kernel;
  cpu_baseline  the CPU oracle timed on this host on a bounded sample (and
                with one BLAS thread on three workloads);
  sclk          the shader clock observed during the timed loop;
  ce / topk / sample / decode_loop
                the cross-entropy, top-k, top-k sampling steps and a
                graph-captured decode loop at the same M;
  construction  archead_build on a seeded dense head against the oracle's
                packer on the same inputs;
  secondary     the same measurement at M=2048 (prefill, MFMA-bound) and the
                other workloads, with fewer steps;
  baselines     the naive group-INT4 and SVD8 + INT4 heads on the same kernels.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA
METRIC = "packed-head tokens/s + HBM GB/s (M=1) and MFMA% (M=2048), 151936x4096 head"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def vtile_bytes(V, d, k, r, g, M):
    """Algorithmic HBM bytes of one vocabulary-tile launch: every packed field
    it reads once (R4 4 bits, sR fp16 per group, A5 5 bits, sA, C8 8 bits, sC),
    X read once, logits written once."""
    per_row = d // 2 + 2 * (d // g) + (5 * k + 7) // 8 + (2 if k else 0) + r + (2 if r else 0)
    return V * per_row + M * d * 2 + M * V * 4


def path_flops(V, d, k, r, M):
    """Algorithmic flops of the whole factored forward (eq 7): 2 M (Vd + Vk + Vr + kd + rd)."""
    return 2 * M * (V * d + V * k + V * r + k * d + r * d)


KERNEL_SOURCES = ("decode.hip", "vtile.hip", "device.hpp", "layout.hpp", "pack.cpp")


def kernel_source_hash():
    """sha256 over the sources that define the vocabulary-tile kernel and the
    layout it reads."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "packed_quantized_lm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(kernel_tag, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_counters.json: FETCH_SIZE and WRITE_SIZE,
    each scaled by what the counter reads for a plain copy of known size).
    None when no summary exists or when it was taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        data = json.load(fh)
    if data.get("source_sha256") != kernel_source_hash():
        return None
    return data.get("hbm_bytes_per_launch")


def _read_sclk_mhz():
    """The current shader clock of each AMD GPU the host exposes, in MHz, from
    the driver's DPM table (the level marked '*'); [] where it cannot be read."""
    import glob
    out = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as fh:
                if fh.read().strip() != "0x1002":
                    continue
            with open(os.path.join(dev, "pp_dpm_sclk")) as fh:
                for line in fh:
                    if "*" in line:
                        out.append(float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz")))
        except (OSError, ValueError, IndexError):
            continue
    return out


class SclkSampler:
    """Polls the shader clock every 2 ms on a host thread while the timed
    region runs (the host thread is otherwise waiting on the GPU)."""

    def __init__(self):
        import threading
        self.samples, self._stop = [], threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            v = _read_sclk_mhz()
            if v:
                self.samples.append(max(v))
            self._stop.wait(0.002)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.array(self.samples)
        return {"source": "pp_dpm_sclk (current DPM level)", "n": int(a.size), "min_mhz": float(a.min()),
                "median_mhz": float(np.median(a)), "max_mhz": float(a.max())}


def measure(name, steps, warmup, copies, path="auto", with_logits=True, extras=True):
    import torch
    from packed_quantized_lm_amd import PackedHead, x_tensor_from_bits
    from packed_quantized_lm_amd.synth import make_config

    t0 = time.time()
    c = make_config(name)
    V, d, k, r, g, M = (c[n] for n in ("V", "d", "k", "r", "g", "M"))
    heads = [PackedHead(c) for _ in range(copies)]
    for h in heads:
        h.reserve(M)
    packed = heads[0].packed_bytes()
    log(f"{name}: generated + loaded {copies} copies in {time.time() - t0:.1f}s")
    X = x_tensor_from_bits(c["X"])
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda") if with_logits else None
    arg = torch.empty((M,), dtype=torch.int32, device="cuda")
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    eva = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for ev in evb + eva:      # torch creates the HIP event on its first record
        ev.record()
    torch.cuda.synchronize()
    for i in range(warmup):
        heads[i % copies].forward_into(X, logits, arg, path=path)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        heads[i % copies].forward_timed(X, logits, arg, evb[i], eva[i], path=path)
    stop.record()
    torch.cuda.synchronize()
    timed_ms = start.elapsed_time(stop)
    kern_ms = np.array([evb[i].elapsed_time(eva[i]) for i in range(steps)])
    # the same steps launched back to back with no events between them
    with SclkSampler() as sclk:
        start.record()
        for i in range(steps):
            heads[i % copies].forward_into(X, logits, arg, path=path)
        stop.record()
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # one copy only ("hot": the previous step's reads may still sit in the
    # memory-side cache); reported beside the rotated figure, never as it
    start.record()
    for i in range(steps):
        heads[0].forward_into(X, logits, arg, path=path)
    stop.record()
    torch.cuda.synchronize()
    hot_ms = start.elapsed_time(stop)
    # and replayed from one HIP graph holding `per_graph` consecutive steps
    # (over the rotated head copies), as a decode loop captured in a graph
    # runs them: no host launch between steps
    graph_ms = None
    per_graph = copies * max(1, 12 // copies)
    try:
        side = torch.cuda.Stream()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=side):
            for i in range(per_graph):
                heads[i % copies].forward_into(X, logits, arg, path=path)
        torch.cuda.synchronize()
        for i in range(max(1, warmup // per_graph)):
            cg.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        start.record()
        for i in range(reps):
            cg.replay()
        stop.record()
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(stop) * steps / (reps * per_graph)
        del cg
    except Exception as e:  # report, do not hide: the direct-launch numbers stand
        log(f"{name}: graph capture failed: {e!r}")
    loop = measure_decode_loop(heads, X, V, d, steps) if extras and M == 1 and path == "auto" else None
    ce = measure_ce(heads, X, V, M, steps, warmup, per_graph, path) if extras else None
    topk = measure_topk(heads, X, V, M, steps, warmup, per_graph, path, logits) if extras else None
    sample = measure_sample(heads, X, V, M, steps, warmup, per_graph, logits) if extras else None
    del heads
    torch.cuda.synchronize()
    # The events around the kernel add their own overhead to each launch.
    # When a step is that one kernel (the single-launch decode path), the
    # back-to-back step time bounds the kernel's duration more tightly; when
    # a step holds several kernels, the step time exceeds the kernel's.  The
    # smaller of the two is an upper bound on the kernel's duration either way.
    kern_s = min(float(np.mean(kern_ms)), total_ms / steps) / 1e3
    vb = vtile_bytes(V, d, k, r, g, M)
    fl = path_flops(V, d, k, r, M)
    best_ms = min(total_ms, graph_ms) if graph_ms is not None else total_ms
    return {
        "workload": name, "V": V, "d": d, "k": k, "r": r, "g": g, "M": M,
        "ms_per_step": best_ms / steps, "tokens_per_s": M / (best_ms / 1e3 / steps),
        "direct_ms_per_step": total_ms / steps,
        "hot_same_copy_ms_per_step": hot_ms / steps,
        "sclk": sclk.summary(),
        "timed_ms_per_step": timed_ms / steps,
        "graph_ms_per_step": None if graph_ms is None else graph_ms / steps,
        "vtile_us_mean": kern_s * 1e6, "vtile_us_p10": float(np.percentile(kern_ms, 10)) * 1e3,
        "vtile_us_p90": float(np.percentile(kern_ms, 90)) * 1e3,
        "packed_bytes": packed, "vtile_bytes": vb,
        "vtile_GBs": vb / kern_s / 1e9, "step_GBs_over_packed": packed / (best_ms / 1e3 / steps) / 1e9,
        "path_TFLOPs": fl / (best_ms / 1e3 / steps) / 1e12, "steps": steps,
        "ce": ce,
        "topk": topk,
        "sample": sample,
        "decode_loop": loop,
    }


def measure_topk(heads, X, V, M, steps, warmup, per_graph, path, logits, K=16):
    """The same step through archead_forward_topk: logits written, then the K
    largest of each row selected from them (the step a top-k sampling decode
    loop runs), back-to-back and from a graph."""
    import torch
    if logits is None:
        logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    copies = len(heads)
    vals = torch.empty((M, K), dtype=torch.float32, device="cuda")
    idx = torch.empty((M, K), dtype=torch.int32, device="cuda")
    step = lambda i: heads[i % copies].forward_topk_into(X, K, logits, vals, idx, path=path)
    return _time_step(step, steps, warmup, per_graph, M, {"K": K})


def measure_sample(heads, X, V, M, steps, warmup, per_graph, logits, K=16, temperature=0.8):
    """The top-k step plus one draw per row at a temperature (a sampling
    decode step), with fixed caller-drawn uniform numbers."""
    import torch
    if logits is None:
        logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    copies = len(heads)
    u = torch.rand((M,), dtype=torch.float32, device="cuda")
    vals = torch.empty((M, K), dtype=torch.float32, device="cuda")
    idx = torch.empty((M, K), dtype=torch.int32, device="cuda")
    samples = torch.empty((M,), dtype=torch.int32, device="cuda")
    step = lambda i: heads[i % copies].forward_sample_into(X, K, temperature, u, logits, vals, idx, samples)
    return _time_step(step, steps, warmup, per_graph, M, {"K": K, "temperature": temperature})


def measure_decode_loop(heads, X0, V, d, steps, K=16, temperature=0.8, per_graph=12):
    """A synthetic sampling decode loop at M = 1: each step runs the packed
    head's forward with top-k sampling (archead_forward_sample), and the drawn
    token picks the next step's hidden state from a seeded bf16 embedding
    table (a row gather standing in for the rest of the model).  per_graph
    steps are captured in one HIP graph (uniform numbers drawn beforehand,
    one per step) and replayed; the head copies rotate as in the other
    measurements.  The graph's token sequence must equal an eager run's."""
    import torch
    copies = len(heads)
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    sig = torch.exp(torch.randn((d,), generator=g, device="cuda"))
    table = (torch.randn((V, d), generator=g, device="cuda") * sig).to(torch.bfloat16)
    u = torch.rand((per_graph, 1), generator=g, device="cuda")
    x = torch.empty((1, d), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((1, V), dtype=torch.float32, device="cuda")
    vals = torch.empty((1, K), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, K), dtype=torch.int32, device="cuda")
    toks = torch.empty((per_graph, 1), dtype=torch.int32, device="cuda")

    def run():
        for t in range(per_graph):
            heads[t % copies].forward_sample_into(x, K, temperature, u[t], logits, vals, idx, toks[t])
            torch.index_select(table, 0, toks[t].long(), out=x)

    x.copy_(X0.view(torch.bfloat16))
    run()
    torch.cuda.synchronize()
    eager = toks.clone()
    side = torch.cuda.Stream()
    cg = torch.cuda.CUDAGraph()
    x.copy_(X0.view(torch.bfloat16))
    torch.cuda.synchronize()
    with torch.cuda.graph(cg, stream=side):
        run()
    x.copy_(X0.view(torch.bfloat16))
    torch.cuda.synchronize()
    cg.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(toks, eager))
    reps = max(1, steps // per_graph)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        cg.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * per_graph)
    del cg, table
    return {"K": K, "temperature": temperature, "steps_per_graph": per_graph, "ms_per_token": ms,
            "tokens_per_s": 1e3 / ms, "graph_tokens_equal_eager": same,
            "step": "archead_forward_sample (forward, top-k selection and draw in the head's launch where it "
                    "applies) + embedding-row gather of the drawn token"}


def _time_step(step, steps, warmup, per_graph, M, extra):
    import torch
    for i in range(warmup):
        step(i)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    direct_ms = start.elapsed_time(stop) / steps
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=side):
            for i in range(per_graph):
                step(i)
        torch.cuda.synchronize()
        cg.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        start.record()
        for i in range(reps):
            cg.replay()
        stop.record()
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(stop) / (reps * per_graph)
        del cg
    except Exception as e:
        log(f"graph capture failed: {e!r}")
    best = min(direct_ms, graph_ms) if graph_ms is not None else direct_ms
    return dict(extra, ms_per_step=best, direct_ms_per_step=direct_ms, graph_ms_per_step=graph_ms,
                tokens_per_s=M / (best / 1e3))


def measure_ce(heads, X, V, M, steps, warmup, per_graph, path):
    """The same step through archead_forward_ce with the log-normaliser and
    cross-entropy reduced inside the tile pass and neither logits nor argmax
    written (the form a perplexity / cross-entropy loop uses): back-to-back
    launches and graph replays over the same rotated head copies."""
    import torch
    copies = len(heads)
    targets = torch.from_numpy(np.random.default_rng(7).integers(0, V, M).astype(np.int32)).cuda()
    lse = torch.empty((M,), dtype=torch.float32, device="cuda")
    nll = torch.empty_like(lse)
    step = lambda i: heads[i % copies].forward_ce_into(X, targets, None, None, lse, nll, path=path)
    for i in range(warmup):
        step(i)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    direct_ms = start.elapsed_time(stop) / steps
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=side):
            for i in range(per_graph):
                step(i)
        torch.cuda.synchronize()
        cg.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        start.record()
        for i in range(reps):
            cg.replay()
        stop.record()
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(stop) / (reps * per_graph)
        del cg
    except Exception as e:
        log(f"forward_ce graph capture failed: {e!r}")
    best = min(direct_ms, graph_ms) if graph_ms is not None else direct_ms
    return {"ms_per_step": best, "direct_ms_per_step": direct_ms, "graph_ms_per_step": graph_ms,
            "tokens_per_s": M / (best / 1e3), "writes": "lse and nll only (no logits, no argmax)"}


def cpu_baseline(name="qwen_m1", budget_s=15.0, one_thread=False):
    """The oracle as it stands (oracle/forward.py, fp64, numpy BLAS) on a
    bounded sample of vocabulary rows of the workload, scaled to tokens/s;
    with one_thread, BLAS limited to one thread."""
    from contextlib import nullcontext

    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import forward, packer
    from packed_quantized_lm_amd.synth import make_config

    c = make_config(name)
    if "W" in c:   # the small case is a dense head: the oracle's packer makes its fields (not timed)
        f, _ = packer.pack(c["W"], c["H"], c["k"], c["r"], c["g"], p=0.75, lam=1e-2)
        c = dict(f, X=c["X"], M=c["M"])
    V, M = c["V"], c["M"]
    block = 8192
    done, t = 0, 0.0
    with threadpool_limits(limits=1) if one_thread else nullcontext():
        # blocks of rows until the budget is spent or the head is done (a head
        # done in under a second is run again, so that the timer resolves it)
        pos = 0
        while t < budget_s and (done < V or t < 1.0):
            rows = np.arange(pos, min(V, pos + block))
            t0 = time.perf_counter()
            forward.forward(c, c["X"], rows=rows)
            t += time.perf_counter() - t0
            done += rows.size
            pos = (pos + rows.size) % V
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    full_s = t * V / done
    return {"value": M / full_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{name}: oracle fp64 forward over {done} vocabulary rows of {V} "
                      f"({t:.2f} s{', one BLAS thread' if one_thread else ''}), scaled to the full head"}


def measure_build(V=32768, d=1024, k=64, r=16, g=128, n_calib=1024, power_iters=8, oversample=16, reps=3):
    """Construction of a packed head (archead_build) from a seeded dense head
    and calibration states, against the oracle's packer on the same inputs
    (exact SVDs, numpy BLAS on the host): the one construction figure the
    pages time."""
    import torch
    from threadpoolctl import threadpool_info

    from oracle import packer
    from packed_quantized_lm_amd import build_head
    from packed_quantized_lm_amd.synth import dense_head

    c = dense_head(V, d, 96, n_calib)
    W = torch.from_numpy(c["W"]).cuda()
    H = torch.from_numpy(c["H"]).cuda()
    args = dict(p=0.75, lam=1e-2, power_iters=power_iters, oversample=oversample, seed=1)
    build_head(W, H, k, r, g, **args)          # warm-up (code loading, first allocations)
    torch.cuda.synchronize()
    gpu = []
    for _ in range(reps):
        t0 = time.perf_counter()
        build_head(W, H, k, r, g, **args)
        torch.cuda.synchronize()
        gpu.append(time.perf_counter() - t0)
    t0 = time.perf_counter()
    packer.pack(c["W"], c["H"], k, r, g, p=0.75, lam=1e-2)
    ora = time.perf_counter() - t0
    threads = max([q.get("num_threads", 1) for q in threadpool_info()] or [1])
    return {"workload": f"dense head V={V} d={d} (rank-96 signal + noise), k={k} r={r} g={g}, "
                        f"{n_calib} calibration rows, p=0.75, lambda=1e-2",
            "gpu_s": float(np.median(gpu)), "gpu_s_all": gpu,
            "gpu_settings": f"randomized SVDs, {power_iters} power iterations, {oversample} extra columns; "
                            "includes copying the fields back to the host",
            "oracle_s": ora, "oracle_cores": int(threads), "oracle": "oracle/packer.py (exact SVDs, fp64)"}


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of nbytes, run steps times: the known
    read and write volume against which the HBM byte counters (FETCH_SIZE,
    WRITE_SIZE) of a profiled run are scaled."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": 4 * n, "steps": steps, "s_per_copy": dt,
                      "GBs_read_plus_write": 8 * n / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--workload", default="qwen_m1")
    ap.add_argument("--path", default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the naive group-INT4 and SVD8+INT4 heads")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the forward step: no cross-entropy or top-k steps and no baseline "
                         "heads (for profiles that must cover the forward's kernels alone)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many bytes "
                         "--steps times (calibration of the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the packed head's "
              "forward is measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return
    from packed_quantized_lm_amd import load_library
    load_library()

    extras = not args.no_extras
    head = measure(args.workload, args.steps, args.warmup, args.copies, path=args.path, extras=extras)
    log(json.dumps(head))
    secondary = []
    if not args.no_secondary:
        for name, steps in [("qwen_m2048", max(5, args.steps // 20)), ("qwen_m32", args.steps),
                            ("large_m8", args.steps)]:
            if name == args.workload:
                continue
            s = measure(name, steps, max(2, args.warmup // 4), args.copies, path=args.path, extras=extras)
            s["mfma_frac"] = s["path_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
            s["hbm_frac"] = s["vtile_GBs"] / HBM_PEAK_GBS
            log(json.dumps(s))
            secondary.append(s)
    # the baseline heads the pages compare against, on the same kernels and
    # the same rotated-copy timing, beside the packed head's step at that M
    baselines = []
    if not args.no_baselines and extras:
        same_m = {head["M"]: head["ms_per_step"]}
        same_m.update({s["M"]: s["ms_per_step"] for s in secondary if s["workload"].startswith("qwen")})
        for name, steps in [("int4_g32_m1", args.steps), ("svd8_int4_m1", args.steps),
                            ("int4_g32_m2048", max(5, args.steps // 20)),
                            ("svd8_int4_m2048", max(5, args.steps // 20))]:
            b = measure(name, steps, max(2, args.warmup // 4), args.copies, path=args.path)
            b["mfma_frac"] = b["path_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
            b["hbm_frac"] = b["vtile_GBs"] / HBM_PEAK_GBS
            b["packed_head_ms_per_step_same_M"] = same_m.get(b["M"])
            log(json.dumps(b))
            baselines.append(b)
    build = None
    if extras:
        build = measure_build()
        log(json.dumps(build))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload)
        log(json.dumps(cpu))
        # one BLAS thread, on the small case, the decode case and the large head
        cpu["one_thread"] = []
        for name in ("tiny", "qwen_m1", "large_m8"):
            one = cpu_baseline(name, budget_s=4.0, one_thread=True)
            log(json.dumps(one))
            cpu["one_thread"].append(dict(one, workload=name))

    traffic = read_traffic("decode_one_launch", args.workload)
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: V={head['V']} d={head['d']} k={head['k']} "
                               f"r={head['r']} g={head['g']} M={head['M']}, 3 rotated copies",
                   "packed_bytes": head["packed_bytes"],
                   "step_GBs_over_packed": head["step_GBs_over_packed"]},
        "roofline": {"bound": "hbm", "achieved": head["vtile_GBs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": head["vtile_GBs"] / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "vocabulary tiles (a2); at M = 1 one launch with a1 and a3",
                     "kernel_us": head["vtile_us_mean"],
                     "bytes_per_launch": head["vtile_bytes"]},
        "cpu_baseline": cpu,
        "sclk": head["sclk"],
        "ce": dict(head["ce"], vs_argmax_step=head["ce"]["ms_per_step"] / head["ms_per_step"]) if extras else None,
        "topk": dict(head["topk"], vs_argmax_step=head["topk"]["ms_per_step"] / head["ms_per_step"]) if extras else None,
        "sample": dict(head["sample"], vs_argmax_step=head["sample"]["ms_per_step"] / head["ms_per_step"])
        if extras else None,
        "decode_loop": dict(head["decode_loop"], vs_argmax_step=head["decode_loop"]["ms_per_token"] / head["ms_per_step"])
        if extras and head.get("decode_loop") else None,
        "construction": build,
        "secondary": secondary,
        "baselines": baselines,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
