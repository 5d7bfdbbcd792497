"""Throughput of batched speculative-sampling verification on one MI355X.

One step = one spec_verify call (softmax statistics, accept / first-reject,
residual or bonus draw, with the early stop: rows after a sequence's first
rejection are not needed) over one batch of the bf16 headline workload:
B=64 sequences, gamma=8 drafted tokens, V=128256, temperature 0.8. Inputs are
seeded synthetic logits already resident in HBM; two input sets alternate so
that every step reads data the previous step did not touch (each set is
279 MB, above the 256 MB last-level cache).

Prints one JSON line: verified draft rows/s (B*gamma per step) with the
library's automatic schedule; the verification kernel's roofline: the
method's algorithmic bytes per launch, every row its definition reads
((2*gamma+1)*B*V*sizeof; the gamma+1 target rows at T == 0), over the
kernel's average launch time against the 8 TB/s peak; beside it the bytes the
chosen schedule needed and their rate (the group-major order skips the bonus
rows of the sequences that stop before them; in two phases the first phase's
row pairs of every sequence are read and the rest only where all of those
were accepted; the early stop reads target and draft rows up to each
sequence's stopping position, plus the bonus row after gamma acceptances);
the same figures for each schedule forced in turn; a plain streaming read of
the same number of bytes (the practical HBM read ceiling); and the fp64 CPU
oracle timed on the host cores, at all cores and at one thread, on bounded
samples of the same workload.

Order on the GPU: the read ceiling, the per-schedule and side legs (each
with its own warm-up), then the headline's W warm-up steps and its K timed
steps, so that the timed steps run at the GPU's steady clocks.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "verified draft rows/sec and achieved HBM GB/s (% of peak) at B=64,γ=8,V=128256"
PEAK_HBM_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "speculative_sampling_verification_05_amd", "csrc", "specverify.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def measured_traffic(kernel, workload):
    """HBM bytes per launch of the verification kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scaled by a plain copy's counts),
    or None if they were taken on another kernel source."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))[f"{kernel}@{workload}"]
        sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec["traffic_bytes"]


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (timing plumbing)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(e.value)
        return out

    def ms(self, a, b):
        f = ctypes.c_float()
        self.hip.hipEventSynchronize(ctypes.c_void_p(b))
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def cpu_model():
    """The host CPU's model name and logical CPU count (from /proc/cpuinfo)."""
    try:
        names = [ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")]
    except OSError:
        names = []
    return {"model": names[0] if names else "unknown", "logical_cpus": len(names) or os.cpu_count()}


def cpu_baseline(inp, seed, sample_b, gpu_tokens=None, gpu_n=None, min_reps=3, min_wall_s=6.0, max_reps=1000,
                 threads=None):
    """The fp64 oracle, as it stands, on the first `sample_b` sequences of the
    workload (same seed, same b indices), timed on the host cores (all of
    them, or `threads`): repeated until at least `min_wall_s` of wall time
    (and `min_reps` runs), median."""
    import oracle
    from oracle.compare import compare_tokens
    wl = inp.wl.scaled(B=sample_b)
    sub = W.Inputs(wl, inp.seed, inp.target[:sample_b], inp.draft[:sample_b], inp.tokens[:sample_b])
    oracle.lib()
    all_threads = oracle.max_threads()
    if threads is not None:
        oracle.set_threads(threads)
    times = []
    res = None
    try:
        used = oracle.max_threads()
        t_start = time.perf_counter()
        while len(times) < max_reps and (len(times) < min_reps or time.perf_counter() - t_start < min_wall_s):
            t0 = time.perf_counter()
            res = oracle.verify(sub.target, sub.draft if wl.T > 0 else None, sub.tokens, wl.dtype, wl.T, seed,
                                diag=True)
            times.append(time.perf_counter() - t0)
    finally:
        oracle.set_threads(all_threads)
    t = float(np.median(times))
    out = {"value": sample_b * wl.gamma / t, "unit": "verified draft rows/s", "cores": used,
           "kind": "oracle",
           "sample": f"first {sample_b} of {inp.wl.B} sequences of the timed workload, median of {len(times)} runs "
                     f"({t:.3f} s per run, fp64, " +
                     ("one thread" if used == 1 else f"OpenMP over sequences, {used} threads") + ")"}
    if gpu_tokens is not None:
        rep = compare_tokens(sub, res, gpu_tokens[:sample_b], gpu_n[:sample_b], seed)
        out["parity_vs_gpu"] = {"hard_failures": len(rep.hard_fail), "near_boundary": rep.mismatches,
                                "draws": rep.draws}
    return out


class StreamRead:
    """The plain streaming-read kernel (libstreamread.so, measurement only)."""

    def __init__(self):
        path = os.path.join(ROOT, "speculative_sampling_verification_05_amd", "libstreamread.so")
        self.lib = ctypes.CDLL(path)
        vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        self.lib.stream_read.argtypes = [vp, i64, i32, u32, vp, vp, vp, vp]
        self.lib.stream_read.restype = ctypes.c_int
        self.lib.stream_read_waves.argtypes = [i64, i32]
        self.lib.stream_read_waves.restype = i64


def launch_floor(hip, nbytes, stream, K=50):
    """The latency floor of a one-launch call that reads `nbytes`: the mean
    duration of an almost empty launch (one wavefront reading 16 bytes) and of
    a plain streaming read of `nbytes` (best range length), each timed with
    HIP events bound to the dispatch."""
    import torch
    sr = StreamRead()
    dev = torch.device("cuda:0")
    buf = torch.empty(max(nbytes, 16) // 4, dtype=torch.int32, device=dev).random_()
    sink = torch.empty(int(sr.lib.stream_read_waves(max(nbytes, 16), 8)), dtype=torch.int32, device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def time_it(nb, cpw):
        for _ in range(5):
            sr.lib.stream_read(buf.data_ptr(), nb, cpw, 0x9E3779B9, sink.data_ptr(), sh, None, None)
        ev = hip.create(2 * K)
        torch.cuda.synchronize()
        for k in range(K):
            sr.lib.stream_read(buf.data_ptr(), nb, cpw, 0x9E3779B9, sink.data_ptr(), sh, ctypes.c_void_p(ev[2 * k]),
                               ctypes.c_void_p(ev[2 * k + 1]))
        torch.cuda.synchronize()
        us = float(np.mean([hip.ms(ev[2 * k], ev[2 * k + 1]) for k in range(K)])) * 1e3
        hip.destroy(ev)
        return us
    empty = time_it(16, 8)
    reads = {cpw: time_it(nbytes, cpw) for cpw in (8, 16, 32)}
    best = min(reads.values())
    return {"empty_launch_us": empty, "plain_read_us": best, "plain_read_bytes": nbytes,
            "plain_read_per_chunks_per_wave_us": {str(k): v for k, v in reads.items()}}


def read_ceiling(hip, nbytes, args, stream, cpws=(8, 16, 24, 32, 64)):
    """A plain read of `nbytes` per launch (the verification's compulsory
    bytes) with 16-byte non-temporal loads, two buffers alternating so that
    every launch reads what the previous one did not touch; every launch
    carries HIP events bound to its dispatch. Returns GB/s per chunks-per-
    wavefront setting and the best."""
    import torch
    sr = StreamRead()
    dev = torch.device("cuda:0")
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_() for _ in range(2)]
    sink = torch.empty(int(sr.lib.stream_read_waves(nbytes, 8)), dtype=torch.int32, device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    K = max(10, min(args.steps, 100))
    for cpw in cpws:
        for s_ in range(3):
            sr.lib.stream_read(bufs[s_ % 2].data_ptr(), nbytes, cpw, 0x9E3779B9, sink.data_ptr(), sh, None, None)
        ev = hip.create(2 * K)
        torch.cuda.synchronize()
        for k in range(K):
            rc = sr.lib.stream_read(bufs[k % 2].data_ptr(), nbytes, cpw, 0x9E3779B9, sink.data_ptr(), sh,
                                    ctypes.c_void_p(ev[2 * k]), ctypes.c_void_p(ev[2 * k + 1]))
            if rc != 0:
                raise RuntimeError(f"stream_read returned {rc}")
        torch.cuda.synchronize()
        us = float(np.mean([hip.ms(ev[2 * k], ev[2 * k + 1]) for k in range(K)])) * 1e3
        hip.destroy(ev)
        out[f"cpw{cpw}"] = {"us": us, "GBps": nbytes / (us * 1e-6) / 1e9}
    best = max(out.values(), key=lambda v: v["GBps"])
    del bufs
    return {"bytes": nbytes, "launches_timed_each": K, "per_chunks_per_wave": out, "best_us": best["us"],
            "best_GBps": best["GBps"], "best_frac": best["GBps"] / PEAK_HBM_GBPS,
            "kernel": "stream_read (16-byte non-temporal loads, contiguous 1 KiB chunks per wavefront)"}


def draft_leg(sv, hip, sets, host0, wl, args, stream):
    """spec_draft_sample over the workload's draft logits, timed like the
    verification: K calls rotating the input sets, every E-th carrying HIP
    events bound to its kernel dispatch. Algorithmic bytes: every row once."""
    import torch
    import oracle
    from oracle.compare import compare_draft
    B, g, V = wl.B, wl.gamma, wl.V
    K, Wm = args.steps, args.warmup
    E = args.event_stride if args.event_stride > 0 else max(1, K // 20)
    esz = 4 if wl.dtype == W.F32 else 2
    out = {}
    one = [s[1][:, 0].contiguous() for s in sets]
    for label, n, logits, ent in (("all_positions", g, [s[1] for s in sets], False),
                                  ("one_position", 1, one, False),
                                  ("all_positions_with_entropy", g, [s[1] for s in sets], True)):
        dev = logits[0].device
        shape = (B, n) if n > 1 else (B,)
        toks = [torch.empty(shape, dtype=torch.int32, device=dev) for _ in logits]
        qs = [torch.empty(shape, dtype=torch.float64, device=dev) for _ in logits]

        def run(step, events=None):
            k = step % len(logits)
            sv.draft_sample(logits[k], wl.T, args.seed + k, out_tokens=toks[k], out_q=qs[k], stream=stream,
                            events=events, want_entropy=ent)
        for s in range(Wm):
            run(s)
        evd = [i for i in range(K) if i % E == 0]
        ev = hip.create(2 * len(evd))
        evmap = {i: (ev[2 * m], ev[2 * m + 1]) for m, i in enumerate(evd)}
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(K):
            run(Wm + s, evmap.get(s))
        end.record(stream)
        torch.cuda.synchronize()
        kms = [hip.ms(ev[2 * m], ev[2 * m + 1]) for m in range(len(evd))]
        hip.destroy(ev)
        ms = start.elapsed_time(end) / K
        nbytes = B * n * V * esz
        k_us = float(np.mean(kms)) * 1e3
        achieved = nbytes / (k_us * 1e-6) / 1e9
        # parity of set 0's first two sequences against the oracle
        run(0)
        torch.cuda.synchronize()
        nb = min(B, 2)
        lg = host0.draft[:nb, :n]
        t = toks[0].cpu().numpy().reshape(B, n)[:nb]
        q = qs[0].cpu().numpy().reshape(B, n)[:nb]
        t0 = time.perf_counter()
        orc = oracle.draft_sample(lg, wl.dtype, wl.T, seed=args.seed)
        t_orc = time.perf_counter() - t0
        rep = compare_draft(lg, wl.dtype, wl.T, orc, t, q, args.seed)
        out[label] = {"rows_per_call": B * n, "ms_per_call": ms, "rows_per_s": B * n / (ms * 1e-3),
                      "kernel_us": k_us, "bytes_per_launch": nbytes, "achieved_GBps": achieved,
                      "frac": achieved / PEAK_HBM_GBPS, "launches_timed": len(kms),
                      "parity_vs_oracle": {"rows": rep.rows, "hard_failures": len(rep.hard_fail),
                                           "near_boundary": rep.boundary},
                      "cpu_baseline": {"value": rep.rows / t_orc, "unit": "rows/s", "cores": oracle.max_threads(),
                                       "kind": "oracle", "sample": f"the first {nb} sequences' rows, one run"}}
    # the floor of the one-position call: a plain read of its bytes (which
    # includes the launch) and an almost empty launch
    fl = launch_floor(hip, B * V * esz, stream)
    fl["one_position_vs_plain_read"] = out["one_position"]["kernel_us"] / fl["plain_read_us"]
    fl["one_position_vs_empty_plus_plain_read"] = out["one_position"]["kernel_us"] / (fl["plain_read_us"] +
                                                                                     fl["empty_launch_us"])
    out["one_position"]["floor"] = fl
    out["kernel"] = "k_draft"
    out["roofline_bound"] = "hbm"
    return out


def expected_accept_leg(sv, sets, wl, args, stream):
    """spec_expected_accept (every position's sum of min(p, q)) on the
    workload: K calls rotating the input sets, timed by stream events around
    the calls (one launch each: the statistics pass, then the overlap)."""
    import torch
    B, g, V = wl.B, wl.gamma, wl.V
    esz = 4 if wl.dtype == W.F32 else 2
    outs = [torch.empty((B, g), dtype=torch.float64, device=sets[0][0].device) for _ in sets]

    def run(step):
        k = step % len(sets)
        sv.expected_accept(sets[k][0], sets[k][1], wl.T, out=outs[k], stream=stream)
    for s_ in range(args.warmup):
        run(s_)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s_ in range(args.steps):
        run(args.warmup + s_)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / args.steps * 1e3
    read = 4 * g * B * V * esz   # statistics of both rows of every pair, then both rows again for the overlap
    minimum = 2 * g * B * V * esz                          # every needed row once
    beta = outs[0].cpu().numpy()
    import oracle
    host = W.make_inputs(wl, args.seed)
    nb = 4
    t0 = time.perf_counter()
    ref = oracle.expected_accept(host.target[:nb], host.draft[:nb], wl.dtype, wl.T)
    t_orc = time.perf_counter() - t0
    err = float(np.nanmax(np.abs(beta[:nb] - ref)))
    return {"us_per_call": us, "positions_per_s": B * g / (us * 1e-6), "bytes_read": read,
            "achieved_GBps": read / (us * 1e-6) / 1e9, "frac": read / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
            "min_bytes": minimum, "mean_beta": float(np.nanmean(beta)), "roofline_bound": "hbm",
            "kernels": ["k_overlap (row statistics of the pairs' target and draft rows, then the overlap sums, one launch)"],
            "parity_vs_oracle": {"positions": nb * g, "max_abs_err": err},
            "cpu_baseline": {"value": nb * g / t_orc, "unit": "positions/s", "cores": oracle.max_threads(),
                             "kind": "oracle", "sample": f"the first {nb} sequences of input set 0, one run"}}


def tree_leg(sv, wl, args, stream):
    """spec_tree_verify (the pages' token-tree heuristic) on seeded trees of
    depth 3 and branching factor 3 ([CSDN] 3.2 uses 3) over the workload's
    vocabulary and dtype: B = 8 trees of 40 nodes, every node's target and
    draft rows (two sets of 164 MB at the headline shape, rotated). Timed by
    stream events around the calls (one launch each)."""
    import torch
    dev = torch.device("cuda:0")
    depth, branch, B = 3, 3, 8
    tdt = torch.float32 if wl.dtype == W.F32 else torch.bfloat16

    def to_dev(a):
        if wl.dtype == W.BF16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
        return torch.from_numpy(a).to(dev)
    sets = []
    for k in range(2):
        tr = W.tree_inputs(B, depth, branch, wl.V, wl.dtype, wl.T, seed=args.seed + 100 + k)
        if k == 0:
            tr0 = tr
        sets.append((to_dev(tr.target), to_dev(tr.draft), torch.from_numpy(tr.parent).to(dev),
                     torch.from_numpy(tr.token).to(dev)))
    N = sets[0][2].shape[1]
    threshold = 0.3
    res = {}

    def run(step):
        t, d, p, tk = sets[step % 2]
        return sv.tree_verify(t, d, p, tk, wl.T, threshold, stream=stream)
    for s_ in range(args.warmup):
        run(s_)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s_ in range(args.steps):
        run(args.warmup + s_)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / args.steps * 1e3
    _, nodes, n = run(0)
    import oracle
    from oracle.compare import compare_tree
    t0 = time.perf_counter()
    orc = oracle.tree_verify(tr0.target, tr0.draft, tr0.parent, tr0.token, wl.dtype, wl.T, threshold)
    t_orc = time.perf_counter() - t0
    near, hard = compare_tree(tr0.target, tr0.draft, tr0.parent, tr0.token, wl.dtype, wl.T, threshold, orc,
                              nodes.cpu().numpy(), n.cpu().numpy())
    nbytes = 2 * B * N * wl.V * (4 if wl.dtype == W.F32 else 2)
    res = {"trees_per_call": B, "nodes_per_tree": N, "depth": depth, "branch": branch, "threshold": threshold,
           "us_per_call": us, "nodes_per_s": B * N / (us * 1e-6), "bytes_per_call": nbytes,
           "achieved_GBps": nbytes / (us * 1e-6) / 1e9, "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
           "mean_accepted_path": float(n.float().mean().item()), "roofline_bound": "hbm",
           "kernels": ["k_tree (row statistics of every node's two rows, then one walking wavefront per tree, one launch)"],
           "mode": "heuristic: not distribution-preserving",
           "parity_vs_oracle": {"trees": B, "hard_failures": len(hard), "near_threshold": len(near)},
           "cpu_baseline": {"value": B / t_orc, "unit": "trees/s", "cores": oracle.max_threads(), "kind": "oracle",
                            "sample": "the trees of input set 0, one run (the oracle walks only the visited nodes' rows)"}}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=W.HEADLINE, choices=list(W.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=2, help="input sets rotated across steps")
    ap.add_argument("--event-stride", type=int, default=0,
                    help="time the kernels of every N-th step of the timed region with HIP events "
                         "(0: steps // 20, so that about 20 launches are timed)")
    ap.add_argument("--vocab", type=int, default=0,
                    help="run the workload at this vocabulary size instead (e.g. 50257: rows whose byte "
                         "length is not a multiple of 16 take the per-element load path)")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--only", choices=("expected_accept", "draft", "tree"), default=None,
                    help="run only this side leg on the workload and print its JSON (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--auto-only", action="store_true",
                    help="time the automatic schedule only (no per-schedule legs; for counter runs)")
    ap.add_argument("--cpu-sample", type=int, default=0, help="sequences in the oracle sample (0: auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the benchmark, run --steps plain device-to-device copies of the "
                         "workload's compulsory byte count (the reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the verification step has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_sampling_verification_05_amd as sv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    if args.vocab:
        wl = wl.scaled(V=args.vocab, name=f"{wl.name.rsplit('_v', 1)[0]}_v{args.vocab}_{wl.name.rsplit('_', 1)[1]}")
    if args.copy_calibration:
        nbytes = wl.compulsory_bytes()
        src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / args.steps * 1e3
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "copies": args.steps,
                          "us_per_copy": us, "GBps_read_plus_write": 2 * nbytes / us / 1e3}), flush=True)
        return
    tdt = torch.float32 if wl.dtype == W.F32 else torch.bfloat16

    def to_dev(a):
        if wl.dtype == W.BF16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
        return torch.from_numpy(a).to(dev)

    t_gen = time.perf_counter()
    sets, host0 = [], None
    for k in range(args.sets):
        inp = W.make_inputs(wl, args.seed + k)
        if k == 0:
            host0 = inp
        sets.append((to_dev(inp.target), to_dev(inp.draft), torch.from_numpy(inp.tokens).to(dev)))
        print(f"[bench] input set {k} ready ({time.perf_counter() - t_gen:.1f} s)", file=sys.stderr, flush=True)
    B, g, V = wl.B, wl.gamma, wl.V
    outs = [(torch.empty((B, g + 1), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
            for _ in range(args.sets)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    dtc = sv.SPEC_F32 if wl.dtype == W.F32 else sv.SPEC_BF16

    def call(step, extras=None):
        tgt, dft, tok = sets[step % args.sets]
        ot, on = outs[step % args.sets]
        rc = sv.verify_raw(tgt.data_ptr(), dft.data_ptr(), tok.data_ptr(), B, g, V, dtc, wl.T,
                           args.seed + (step % args.sets), ot.data_ptr(), on.data_ptr(), sh, extras)
        if rc != 0:
            raise RuntimeError(f"spec_verify returned {rc}: {sv.last_error()}")

    hip = HipEvents()
    K, Wm = args.steps, args.warmup
    if args.only:
        leg = {"expected_accept": lambda: expected_accept_leg(sv, sets, wl, args, stream),
               "draft": lambda: draft_leg(sv, hip, sets, host0, wl, args, stream),
               "tree": lambda: tree_leg(sv, wl, args, stream)}[args.only]()
        print(json.dumps({"only": args.only, "workload": wl.name, args.only: leg}), flush=True)
        return
    # the plain streaming read of the same byte count first: the practical
    # ceiling, measured on an idle GPU, which also brings it to its steady
    # clocks before the verification's warm-up and timed steps
    rc_ = None if args.no_read_ceiling else read_ceiling(hip, wl.compulsory_bytes(), args, stream)
    if rc_ is not None:
        print(f"[bench] read ceiling {rc_['best_GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    def timed(make_extras):
        """K steps of the call (the timed region, bracketed by stream events);
        every E-th step carries two HIP events bound to its kernel dispatch
        (start and end of the verification kernel), which time the kernel
        inside the timed region without adding packets to the stream."""
        evd = [i for i in range(K) if i % E == 0]
        ev = hip.create(2 * len(evd))
        ex = {}
        for n, i in enumerate(evd):
            e = make_extras()
            e.events[0] = ev[2 * n]
            e.events[1] = ev[2 * n + 1]
            ex[i] = e
        plain = make_extras()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(K):
            call(Wm + s, ex.get(s, plain))
        end.record(stream)
        torch.cuda.synchronize()
        kms = [hip.ms(ev[2 * n], ev[2 * n + 1]) for n in range(len(evd))]
        hip.destroy(ev)
        return start.elapsed_time(end) / K, kms, evd

    def with_schedule(sched):
        def make():
            e = sv.Extras()
            e.schedule = sched
            return e
        return make

    E = args.event_stride if args.event_stride > 0 else max(1, K // 20)

    # bytes the early-stopping algorithm needs for each input set (its outputs
    # are the same on every step: same inputs, same seed)
    def needed_bytes(n):
        row = V * (4 if wl.dtype == W.F32 else 2)
        if wl.T == 0.0:
            rows = np.where(n < 0, g + 1, np.minimum(n, g) + 1)
        else:
            rows = np.where((n < 0) | (n >= g), 2 * g + 1, 2 * (n + 1))
        return int(rows.sum()) * row

    # bytes the group-major order needs at T > 0 with no per-row outputs asked
    # for: every row but the bonus row, which only the sequences that accept
    # every draft token read (an invalid sequence is counted as reading it)
    def group_bytes(n):
        if wl.T == 0.0:
            return wl.compulsory_bytes()
        row = V * (4 if wl.dtype == W.F32 else 2)
        return int(2 * g * B + np.sum((n < 0) | (n >= g))) * row

    # bytes the group-major order in two phases needs at T > 0: the first p0
    # row pairs of every sequence, the other pairs only for the sequences that
    # accept all of those, and the bonus row for those that accept every
    # token (p0 as the header states it; an invalid sequence is counted as
    # reading every row)
    p0 = 0 if g < 2 else max(1, min((3 * g + 4) // 8, g - 1))

    def two_phase_bytes(n):
        if wl.T == 0.0 or p0 == 0:
            return group_bytes(n)
        row = V * (4 if wl.dtype == W.F32 else 2)
        bad = n < 0
        rows = 2 * p0 + np.where(bad | (n >= p0), 2 * (g - p0), 0) + np.where(bad | (n >= g), 1, 0)
        return int(rows.sum()) * row

    set_bytes, set_group_bytes, set_two_bytes = [], [], []
    for k in range(args.sets):
        call(k)
        torch.cuda.synchronize()
        n_k = outs[k][1].cpu().numpy()
        set_bytes.append(needed_bytes(n_k))
        set_group_bytes.append(group_bytes(n_k))
        set_two_bytes.append(two_phase_bytes(n_k))
    compulsory = wl.compulsory_bytes()
    # the metric's formula, (2 gamma + 1) B V s; at T == 0 the draft rows are
    # never read, so the compulsory bytes are the target rows alone
    formula_bytes = (2 * g + 1) * B * V * wl.elem_bytes

    def algo_bytes(sched, steps):
        """Algorithmic bytes of each listed step: the early stop needs the rows
        up to each sequence's stopping position; the group-major order every
        row but the bonus rows of the sequences that stop before it; the
        position-major order without the early stop every row (the compulsory
        bytes)."""
        if sched == sv.SCHEDULE_EARLY_STOP:
            return [set_bytes[(Wm + i) % args.sets] for i in steps]
        if sched == sv.SCHEDULE_GROUP:
            return [set_group_bytes[(Wm + i) % args.sets] for i in steps]
        if sched == sv.SCHEDULE_GROUP_TWO_PHASE:
            return [set_two_bytes[(Wm + i) % args.sets] for i in steps]
        return [compulsory for _ in steps]

    names = {sv.SCHEDULE_GROUP: "group", sv.SCHEDULE_EARLY_STOP: "early_stop", sv.SCHEDULE_POSITION: "position",
             sv.SCHEDULE_GROUP_TWO_PHASE: "two_phase"}
    rows_per_step = B * g
    schedules = {}
    # (at T == 0 every schedule but GROUP is the position-major order with the early stop)
    legs = () if args.auto_only else ((sv.SCHEDULE_GROUP, sv.SCHEDULE_EARLY_STOP) if wl.T == 0.0 else
                                      (sv.SCHEDULE_GROUP, sv.SCHEDULE_GROUP_TWO_PHASE, sv.SCHEDULE_EARLY_STOP,
                                       sv.SCHEDULE_POSITION))
    for sched in legs:
        ms_s, km_s, ev_s = timed(with_schedule(sched))
        a_s = compulsory / (float(np.mean(km_s)) * 1e-3) / 1e9
        r_s = float(np.sum(algo_bytes(sched, ev_s))) / (float(np.sum(km_s)) * 1e-3) / 1e9
        schedules[names[sched]] = {"ms_per_step": ms_s, "kernel_us": float(np.mean(km_s)) * 1e3,
                                   "rows_per_s": rows_per_step / (ms_s * 1e-3), "achieved_GBps": a_s,
                                   "frac": a_s / PEAK_HBM_GBPS,
                                   "needed_bytes_per_launch": float(np.mean(algo_bytes(sched, ev_s))),
                                   "needed_GBps": r_s}

    # the draft-side sampler on the same workload's draft logits: all B x gamma
    # rows per call, and one position (B rows, one autoregressive step)
    draft = None if args.auto_only or wl.T == 0.0 else draft_leg(sv, hip, sets, host0, wl, args, stream)
    overlap = None if args.auto_only or wl.T == 0.0 else expected_accept_leg(sv, sets, wl, args, stream)
    tree = None if args.auto_only or wl.T == 0.0 else tree_leg(sv, wl, args, stream)

    # the headline: the automatic schedule, W warm-up steps, then exactly K
    # timed steps (after the legs above, so that the GPU is at its steady clocks)
    for s in range(Wm):
        call(s)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({Wm} steps)", file=sys.stderr, flush=True)
    ms_per_step, k_ms, evd = timed(with_schedule(sv.SCHEDULE_AUTO))

    # the same steps with no events at all (reported beside the timed value)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(K):
        call(Wm + s)
    end.record(stream)
    torch.cuda.synchronize()
    ms_plain = start.elapsed_time(end) / K

    auto = sv.auto_schedule(B, g, V, dtc, wl.T)
    kname = "k_group" if auto in (sv.SCHEDULE_GROUP, sv.SCHEDULE_GROUP_TWO_PHASE) else "k_verify"
    k_bytes = algo_bytes(auto, evd)
    rows_per_step = B * g
    value = rows_per_step / (ms_per_step * 1e-3)
    k_avg_ms = float(np.mean(k_ms))
    # the roofline's algorithmic bytes per launch: every row the method's
    # definition reads, (2 gamma + 1) B V s (the target rows alone at T == 0),
    # whatever the schedule skips; the bytes the chosen schedule needed and
    # their rate are reported beside them
    achieved = compulsory / (k_avg_ms * 1e-3) / 1e9
    needed_rate = float(np.sum(k_bytes)) / (float(np.sum(k_ms)) * 1e-3) / 1e9

    traffic = measured_traffic(kname, wl.name)
    # one validation of the outputs of set 0 against the oracle (outside the timed region)
    call(0)
    torch.cuda.synchronize()
    gpu_t = outs[0][0].cpu().numpy()
    gpu_n = outs[0][1].cpu().numpy()
    n_hist = np.bincount(gpu_n[gpu_n >= 0], minlength=g + 1).tolist()

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "verified draft rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: fp32 exponentials, fp64 sums and comparisons
        # (the logits' storage type is config.logits)
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "gamma": g, "V": V, "temperature": wl.T,
                   "logits": W.DTYPE_NAMES[wl.dtype], "input_sets": args.sets},
        "kernel_us": {kname: k_avg_ms * 1e3},
        "ms_per_step_no_events": ms_plain,
        "event_stride": E,
        "schedule": names[auto],
        "accepted_hist": n_hist,
        "needed_bytes_per_set": set_bytes,
        "group_bytes_per_set": set_group_bytes,
        "two_phase_bytes_per_set": set_two_bytes,
        "compulsory_bytes": compulsory,
        "metric_formula_bytes": formula_bytes,
        # the same step counted in sequences and in logit rows read (other
        # readings of "verified rows"), and the HBM bytes the counters measured
        # per launch (re-read of row k included) over the kernel's time
        "sequences_per_s": B / (ms_per_step * 1e-3),
        "logit_rows_per_s": ((g + 1) if wl.T == 0.0 else (2 * g + 1)) * B / (ms_per_step * 1e-3),
        "actual_GBps": (traffic / (k_avg_ms * 1e-3) / 1e9) if traffic else None,
        # the metric's own reading: its formula bytes over the kernel's time
        # (above the rate on the bytes read when the schedule skips rows)
        "metric_formula_GBps": formula_bytes / (k_avg_ms * 1e-3) / 1e9,
        "metric_formula_frac": formula_bytes / (k_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "bytes_per_launch": compulsory, "avg_launch_us": k_avg_ms * 1e3,
                     "launches_timed": len(k_ms),
                     "needed_bytes_per_launch": float(np.mean(k_bytes)), "needed_GBps": needed_rate,
                     "needed_frac": needed_rate / PEAK_HBM_GBPS},
        "schedules": schedules,
    }
    if draft is not None:
        result["draft_sampler"] = draft
    if overlap is not None:
        result["expected_accept"] = overlap
    if tree is not None:
        result["tree_verify"] = tree
    if rc_ is not None:
        rc_["verification_kernel_vs_ceiling"] = (float(np.mean(k_bytes)) / (k_avg_ms * 1e-3) / 1e9) / rc_["best_GBps"]
        result["read_ceiling"] = rc_
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or min(B, 64)
        cb = cpu_baseline(host0, args.seed, sample, gpu_t, gpu_n)
        cb["one_thread"] = cpu_baseline(host0, args.seed, min(sample, 8), gpu_t, gpu_n, threads=1)
        cb["host_cpu"] = cpu_model()
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
