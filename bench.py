"""Benchmark of the SDM forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]
    python bench.py --copy-calibration      # plain 1 GiB device copy, for scaling HBM counters
    python bench.py --op sdm_bwd [--workload 1]   # the backward
    python bench.py --op topk               # the product-key top-k

A step is one sdm_fwd call over the whole workload (every chunk step of every stream)
with all inputs resident in HBM. The default workload is config 4 (64 streams x 4096
tokens, chunk 256, head_dim 256, 131072 bf16 rows per stream, 256 write and 256 read
slots per token), the largest single-GPU configuration and the one the throughput metric
is quoted on. Each timed step is bracketed by HIP events on the library's stream; before
it, outside the timed region, the bank is restored from a pristine copy (the op advances
it in place) and the 256 MB last-level cache (MALL) is flushed by writing 1 GiB of
scratch, so every step starts cold from the same state. `ms_per_step` is the median over
the K steps (the mean is reported beside it, and a warm median taken without the flush).
Prints one JSON line: tokens/s, the per-kernel breakdown from HIP events recorded by the
library on its stream, the roofline of the dominant kernel against the 8 TB/s datasheet
peak and against a device copy measured in the same run, and the CPU oracle's throughput
on the host as a reference.

The roofline's `traffic` (HBM bytes per Phase-2 launch) comes from the committed counter
summary profiles/traffic_<workload>.md (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by the
same counters' reading for a plain copy) and is reported only while the Phase-2 sources
hash to the value recorded there; otherwise it is null.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, datasheet
# kernel-boundary intervals of sdm_exec.events; the first is the partitioned Phase-1 kernel
# plus the sort (which skips the chunks the partitioned kernel handled), or the fused kernel
KERNELS = ("p1_partition_sort", "p1_groups", "p1_reads", "p1_gram_cold", "p1_gram_hot", "wy_solve", "phase2")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="4", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--overlap", action="store_true",
                    help="also time a loop in which batch k+1's Phase 1 overlaps batch k's Phase 2 on a second "
                         "stream (reported beside the headline; the bank is then advanced in place)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 launches)")
    ap.add_argument("--op", default="sdm_fwd", choices=("sdm_fwd", "sdm_bwd", "topk"),
                    help="sdm_fwd: the memory op (default); sdm_bwd: its backward on the workload's shapes "
                         "with a float32 bank; topk: the product-key top-k that selects its slots, on the "
                         "workload TOPK_WORKLOAD")
    return ap.parse_args()


# The product-key top-k workload: the write-slot selection of workload 2's tokens (32 x 4096
# rows), its 16384 slots as two factors of 128, k = W = 32, bfloat16 scores ~ N(0, 1).
TOPK_WORKLOAD = dict(rows=32 * 4096, factors=(128, 128), k=32, dtype="bf16", seed=20261202)


def bench_topk(args):
    import torch
    from chunked_sparse_delta_amd import product_key_topk
    from oracle import product_key_topk as pko
    w = TOPK_WORKLOAD
    D, kk = sum(w["factors"]), min(w["k"], int(np.prod(w["factors"])))
    rng = np.random.default_rng(w["seed"])
    x32 = rng.standard_normal((w["rows"], D), dtype=np.float32)
    bits = workloads.round_bf16_bits(x32)
    dev = torch.device("cuda:0")
    raw = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    for _ in range(args.warmup):
        product_key_topk(raw, w["factors"], w["k"])
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        product_key_topk(raw, w["factors"], w["k"])
    e1.record(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = e0.elapsed_time(e1) / args.steps
    es = 2
    alg = w["rows"] * (D * es + kk * (es + 8))   # scores in, values and slot ids out
    gbs = alg / (kern_ms * 1e-3) / 1e9
    name = f"pktopk_rows{w['rows']}_f{'x'.join(map(str, w['factors']))}_k{w['k']}_{w['dtype']}"
    res = {
        "metric": "product-key top-k rows/sec at 1 MI355X", "value": round(w["rows"] * args.steps / elapsed, 1),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1000.0 * elapsed / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "rows": w["rows"], "factors": list(w["factors"]), "k": w["k"],
                   "score_dtype": w["dtype"]},
        "kernel_ms": {"topk": round(kern_ms, 5)},
        "roofline": {"bound": "hbm", "kernel": "topk", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(alg),
                     "note": "in-LDS sorts per row bound the kernel; the bytes are what the rows must move"},
    }
    if not args.no_cpu_baseline:
        sample = workloads.bf16_bits_to_f32(bits[:256])
        reps, c0 = 0, time.perf_counter()
        while time.perf_counter() - c0 < args.cpu_seconds:
            pko.product_key_topk(sample, w["factors"], w["k"], bf16=True)
            reps += 1
        el = time.perf_counter() - c0
        res["cpu_baseline"] = {"value": round(256 * reps / el, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"the first 256 rows x {reps} passes of the Python oracle, 1 thread, {el:.1f} s"}
    print(json.dumps(res), flush=True)


PHASE2_SOURCES = ("chunked_sparse_delta_amd/csrc/phase2.hip", "chunked_sparse_delta_amd/csrc/common.h")


def phase2_source_hash() -> str:
    h = hashlib.sha256()
    for rel in PHASE2_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


BWD_SOURCES = ("chunked_sparse_delta_amd/csrc/backward.hip", "chunked_sparse_delta_amd/csrc/backward.h")


def bwd_source_hash() -> str:
    h = hashlib.sha256()
    for rel in BWD_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, field: str = "phase2_source_sha256", current=None):
    """HBM bytes per launch of the dominant kernel from profiles/traffic_<workload>.md, if it
    was taken on the current sources of that kernel (Phase 2, or the backward sweep); else
    None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", open(path).read(), flags=re.M))
    if fields.get(field) != (current if current is not None else phase2_source_hash()):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = 1 << 28   # 1 GiB of float32
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": 4 * n, "copy_bytes_written_per_launch": 4 * n}), flush=True)


def chunk_stats(inp: dict, wl) -> dict:
    """Exact distinct-row counts per live chunk: U (rows read: write or read slots) and
    U_w (rows written), summed over chunks, plus live token rows."""
    P, T, C, M = wl.P, wl.T, wl.C, wl.M
    valid = np.asarray(inp["valid"], dtype=np.int64)
    U = Uw = live = 0
    for p in range(P):
        nv = int(valid[p])
        if nv == 0:
            continue
        tok_chunk = (np.arange(nv) // C).astype(np.int64)
        kw = inp["k_idx"][p, :nv].astype(np.int64)
        kr = inp["q_idx"][p, :nv].astype(np.int64)
        wkeys = (tok_chunk[:, None] * M + kw).ravel()
        rkeys = (tok_chunk[:, None] * M + kr).ravel()
        uw = np.unique(wkeys)
        Uw += uw.size
        U += np.union1d(uw, np.unique(rkeys)).size
        live += nv
    return dict(U=int(U), Uw=int(Uw), live_tokens=int(live))


def hip_runtime():
    """The HIP runtime already loaded by torch (one runtime per process)."""
    maps = open("/proc/self/maps").read()
    paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so[.\d]*)", maps)))
    lib = ctypes.CDLL(paths[0] if paths else "libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def to_torch(inp: dict, device) -> dict:
    import torch
    dt = inp["dtype"]

    def bank_dtype(a):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(bank=bank_dtype(inp["bank"]), k_idx=torch.from_numpy(inp["k_idx"]).to(device),
                q_idx=torch.from_numpy(inp["q_idx"]).to(device), k_val=bank_dtype(inp["k_val"]),
                q_val=bank_dtype(inp["q_val"]), v=bank_dtype(inp["v"]), beta=torch.from_numpy(inp["beta"]).to(device),
                log_decay=torch.from_numpy(inp["log_decay"]).to(device),
                valid=torch.from_numpy(np.ascontiguousarray(inp["valid"], dtype=np.int32)).to(device))


BWD_KERNELS = ("bwd_lead", "bwd_sweep", "bwd_reduce")


def bench_bwd(args):
    """One step = one sdm_bwd call over the whole workload (the config's shapes and bank
    dtype): the replay of the forward, the reverse sweep and the reduction. The bank comes
    back bit for bit after each call; grad_bank is carried from call to call (in/out), which
    changes values, not work."""
    import torch
    from chunked_sparse_delta_amd import BWD_TIMING_EVENTS, bwd_workspace_bytes, sdm_bwd
    wl = workloads.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    name = workloads.workload_name(wl).replace("sdm_fwd_", "sdm_bwd_", 1)
    print(f"bench: generating workload {name}", file=sys.stderr, flush=True)
    inp = workloads.generate(wl)
    gr = workloads.grad_inputs(wl, 0)
    t = to_torch(inp, dev)
    if wl.dtype == "bf16":
        bits = workloads.round_bf16_bits(gr["grad_out"])
        gr["grad_out"] = workloads.bf16_bits_to_f32(bits)
        go = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        go = torch.from_numpy(gr["grad_out"]).to(dev)
    gbank = torch.from_numpy(gr["grad_bank"]).to(dev)
    ws = torch.empty(bwd_workspace_bytes(wl.P, wl.T, wl.W, wl.R, wl.hd, wl.M, t["bank"].dtype), dtype=torch.uint8,
                     device=dev)
    hip = hip_runtime()
    nev = BWD_TIMING_EVENTS
    ev_sets = []
    for _ in range(args.steps):
        arr = (ctypes.c_void_p * nev)()
        for k in range(nev):
            ev = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[k] = ev.value
        ev_sets.append(arr)

    def step(events=None):
        sdm_bwd(t["bank"], t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], go,
                grad_bank=gbank, valid_tokens=t["valid"], workspace=ws, events=events)

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"bench: {args.steps} instrumented steps for the per-kernel times", file=sys.stderr, flush=True)
    for k in range(args.steps):
        step(ev_sets[k])
    torch.cuda.synchronize()
    per = np.zeros((args.steps, nev - 1))
    for k, arr in enumerate(ev_sets):
        for j in range(nev - 1):
            ms = ctypes.c_float()
            hip.hipEventElapsedTime(ctypes.byref(ms), arr[j], arr[j + 1])
            per[k, j] = ms.value
        for j in range(nev):
            hip.hipEventDestroy(arr[j])
    kern_ms = dict(zip(BWD_KERNELS, per.mean(axis=0).round(5).tolist()))

    # Algorithmic bytes of the sweep: what any backward of this design-independent form must
    # move, plus the saved rows an exact restore needs. Per call, the bank read once and the
    # bank gradient read and written once (float32); per live token, v and grad_out read
    # once (bank dtype), grad_v written (float32), slot ids and weights read, gates and beta
    # read, their gradients written (float32), and each write entry's row saved and read back
    # once (float32 working values).
    # the library's slice width (shapes only): 4 columns when a token has at most 128 slots of
    # each kind, else the widest power of two up to 64 that still gives 256 workgroups
    S = 4
    if max(wl.W, wl.R) > 128:
        while S < 64 and S < wl.hd:
            S <<= 1
        while S > 4 and wl.P * (-(-wl.hd // S)) < 256:
            S >>= 1
    valid = np.asarray(inp["valid"], dtype=np.int64)
    tokens = int(valid.sum())
    es = 4 if wl.dtype == "f32" else 2
    per_token = (wl.hd * (2 * es + 4) + (wl.W + wl.R) * (4 + es) + 4 * wl.G + 4 + 4 * (wl.W + wl.R + wl.G + 1)
                 + 2 * wl.W * wl.hd * 4)
    sweep_bytes = wl.P * wl.M * wl.hd * (es + 8) + tokens * per_token
    gbs = sweep_bytes / (kern_ms["bwd_sweep"] * 1e-3) / 1e9
    res = {
        "metric": "SDM bwd tokens/sec at 1 MI355X", "value": round(tokens * args.steps / elapsed, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1000.0 * elapsed / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "streams": wl.P, "tokens": wl.T, "head_dim": wl.hd, "rows": wl.M,
                   "write_slots": wl.W, "read_slots": wl.R, "bank_dtype": wl.dtype, "ids": wl.ids},
        "kernel_ms": kern_ms,
        "roofline": {"bound": "hbm", "kernel": "bwd_sweep", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5),
                     "traffic": measured_traffic(f"bwd_{args.workload}", "bwd_source_sha256", bwd_source_hash()),
                     "bytes_per_launch": int(sweep_bytes), "slice_columns": S,
                     "note": "token-sequential per column slice: bound by the latency of each token's "
                             "dependent loads and barriers, not by bandwidth"},
    }
    if not args.no_cpu_baseline:
        import oracle
        f = oracle.as_f64_inputs(inp)
        threads = max(1, min(wl.P, os.cpu_count() or 1, 16))
        oracle.token_loop_backward(f, gr["grad_out"], gr["grad_bank"], threads=threads)
        reps, c0 = 0, time.perf_counter()
        while True:
            oracle.token_loop_backward(f, gr["grad_out"], gr["grad_bank"], threads=threads)
            reps += 1
            el = time.perf_counter() - c0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": round(reps * tokens / el, 1), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle", "sample": f"the whole workload x {reps} passes of the fp64 "
                                                           f"backward oracle, {threads} threads, {el:.1f} s"}
    print(json.dumps(res), flush=True)


def cpu_baseline(inp: dict, wl, seconds: float, streams_total: int, twin: str = "") -> dict:
    import oracle
    f = oracle.as_f64_inputs(inp)
    threads = max(1, min(wl.P, os.cpu_count() or 1, 16))
    tokens = int(np.sum(inp["valid"]))
    oracle.token_loop(f, threads=threads)      # build / warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.token_loop(f, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # one thread on the sample's first stream alone (its own bank: no other stream's rows copied)
    f1 = {k: np.ascontiguousarray(v[:1]) for k, v in f.items()}
    tok1 = int(np.sum(f1["valid"]))
    oracle.token_loop(f1, threads=1)
    reps1, t1 = 0, time.perf_counter()
    while True:
        oracle.token_loop(f1, threads=1)
        reps1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 3:
            break
    return {"value": reps * tokens / el, "unit": "tokens/s", "cores": threads, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{wl.P} of the workload's {streams_total} streams{twin} ({tokens} valid tokens) x {reps} "
                      f"passes of the fp64 token loop, {threads} threads, {el:.1f} s",
            "one_thread": {"value": reps1 * tok1 / el1, "unit": "tokens/s",
                           "sample": f"stream 0 of that sample ({tok1} valid tokens) x {reps1} passes, 1 thread, "
                                     f"{el1:.1f} s"}}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on exactly one GPU (the forward shards with no exchange across "
              "streams or columns, but no multi-GPU path is built); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.op == "topk":
        bench_topk(args)
        return
    if args.op == "sdm_bwd":
        bench_bwd(args)
        return
    import torch
    from chunked_sparse_delta_amd import TIMING_EVENTS, plan, sdm_fwd, sdm_fwd_phase1, sdm_fwd_phase2, workspace_bytes

    wl = workloads.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    print(f"bench: generating workload {workloads.workload_name(wl)}", file=sys.stderr, flush=True)
    inp = workloads.generate(wl)
    stats = chunk_stats(inp, wl)
    t = to_torch(inp, dev)
    es = 4 if wl.dtype == "f32" else 2
    torch.cuda.synchronize()

    ws = torch.empty(workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 0), dtype=torch.uint8, device=dev)
    out = torch.empty((wl.P, wl.T, wl.hd), dtype=t["bank"].dtype, device=dev)
    bank = t["bank"]
    hip = hip_runtime()
    nev = TIMING_EVENTS
    ev_sets = []
    for _ in range(args.steps):
        arr = (ctypes.c_void_p * nev)()
        for k in range(nev):
            ev = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[k] = ev.value
        ev_sets.append(arr)

    fargs = (t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"])
    pristine = bank.clone()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # 4x the 256 MB MALL
    stream = torch.cuda.current_stream()

    def step(events=None):
        sdm_fwd(bank, *fargs, chunk=wl.C, valid_tokens=t["valid"], out=out, workspace=ws, events=events)

    def prepare(cold: bool):
        # outside the timed region: the pristine bank, and (cold) a MALL flushed by 1 GiB of writes
        bank.copy_(pristine)
        if cold:
            flush.fill_(1)

    def timed_steps(K: int, cold: bool) -> np.ndarray:
        """K calls, each from the pristine bank, timed by HIP events on the call's stream."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for k in range(K):
            prepare(cold)
            evs[k][0].record(stream)
            step()
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) for e0, e1 in evs])

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        prepare(True)
        step()
    torch.cuda.synchronize()
    print(f"bench: timing {args.steps} cold steps", file=sys.stderr, flush=True)
    t_wall = time.perf_counter()
    cold_ms = timed_steps(args.steps, True)
    t_wall = time.perf_counter() - t_wall
    print(f"bench: timing {args.steps} warm steps", file=sys.stderr, flush=True)
    warm_ms = timed_steps(args.steps, False)
    print(f"bench: {args.steps} instrumented steps for the per-kernel times", file=sys.stderr, flush=True)
    for k in range(args.steps):
        prepare(True)
        step(ev_sets[k])
    torch.cuda.synchronize()
    per = np.zeros((args.steps, nev - 1))
    for k, arr in enumerate(ev_sets):
        for j in range(nev - 1):
            ms = ctypes.c_float()
            hip.hipEventElapsedTime(ctypes.byref(ms), arr[j], arr[j + 1])
            per[k, j] = ms.value
        for j in range(nev):
            hip.hipEventDestroy(arr[j])
    kern_ms = dict(zip(KERNELS, np.median(per, axis=0).round(5).tolist()))

    # The achievable bandwidth of a plain device copy (1 GiB read + 1 GiB written), same run.
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    copy_ms = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    copy_gbs = 2 * src.numel() / (float(np.median(copy_ms[1:])) * 1e-3) / 1e9
    del src, dst

    overlapped_ms = None
    if args.overlap:
        overlapped_ms = overlapped_loop(args, wl, bank, fargs, ws, out, t, sdm_fwd_phase1, sdm_fwd_phase2)

    tokens = stats["live_tokens"]
    ms_step = float(np.median(cold_ms))
    value = tokens / (ms_step * 1e-3)
    row = es * wl.hd
    p2_bytes = row * (stats["U"] + stats["Uw"]) + row * tokens + row * wl.P * wl.T
    entry_bytes = tokens * (wl.W * (4 + es + 4) + wl.R * (4 + es) + 4)
    path_bytes = p2_bytes + entry_bytes
    dom = max(kern_ms, key=kern_ms.get)
    if dom == "phase2":
        achieved = p2_bytes / (kern_ms["phase2"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "phase2", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
                "bytes_per_launch": int(p2_bytes), "copy_gbs": round(copy_gbs, 1),
                "frac_of_copy": round(achieved / copy_gbs, 4)}
    else:
        roof = {"bound": "alu", "kernel": dom, "achieved": None, "peak": None, "unit": None, "frac": None,
                "traffic": None, "note": "dominant kernel is a Phase-1 kernel; see kernel_ms"}
    path_gbs = path_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "SDM fwd tokens/sec at 1 MI355X; achieved HBM GB/s fraction of peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": workloads.workload_name(wl), "streams": wl.P, "tokens": wl.T, "chunk": wl.C,
                   "head_dim": wl.hd, "rows_per_stream": wl.M, "bank_dtype": wl.dtype, "W": wl.W, "R": wl.R,
                   "valid_tokens": tokens, "distinct_rows_read": stats["U"], "rows_written": stats["Uw"]},
        "timing": ("median of K sdm_fwd calls, each timed by HIP events on its stream, the bank restored from "
                   "a pristine copy and the MALL flushed (1 GiB written) before each call, outside the timed "
                   "region; arithmetic in float32 (bank dtype in config)"),
        "ms_per_step_mean": round(float(np.mean(cold_ms)), 4),
        "ms_per_step_warm": round(float(np.median(warm_ms)), 4),
        "wall_s_timed_loop": round(t_wall, 3),
        "kernel_ms": kern_ms,
        "plan": plan(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, wl.M, bank.dtype),
        "roofline": roof,
        "path_hbm": {"algorithmic_bytes": int(path_bytes), "achieved": round(path_gbs, 1), "unit": "GB/s",
                     "frac": round(path_gbs / HBM_PEAK_GBS, 4), "frac_of_copy": round(path_gbs / copy_gbs, 4)},
    }
    if overlapped_ms is not None:
        res["ms_per_step_overlapped"] = round(overlapped_ms, 4)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        sample = inp
        host = os.cpu_count() or 1
        if wl.P > min(16, host) or wl.name in ("4", "4p"):
            keep = list(range(min(wl.P, host, 16)))
            # config 4 overflows as drawn; its finite twin 4p has the same shapes and cost
            sample = workloads.generate(workloads.CONFIGS["4p"] if wl.name == "4" else wl, streams=keep)
        twin = " (of its finite twin 4p: the same shapes and ids, weights / sqrt(W))" if wl.name == "4" else ""
        res["cpu_baseline"] = cpu_baseline(sample, wl.replace(P=len(sample["valid"])), args.cpu_seconds, wl.P, twin)
    print(json.dumps(res), flush=True)


def overlapped_loop(args, wl, bank, fargs, ws, out, t, sdm_fwd_phase1, sdm_fwd_phase2) -> float:
    """ms per step of a loop in which batch k+1's Phase 1 runs on a second stream (and a
    second workspace) while batch k's Phase 2 runs on the first; every step still runs both
    phases in full, and the bank advances in place from step to step. Phase 1 of k+1 waits
    for Phase 2 of k-1 (which read the workspace it reuses) and then for a one-element marker
    kernel on its own stream, so that Phase 2's workgroups are placed first."""
    import torch
    dev = bank.device
    ws_pair = [ws, torch.empty_like(ws)]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    p1_done = [torch.cuda.Event(), torch.cuda.Event()]
    p2_done = [torch.cuda.Event(), torch.cuda.Event()]
    marker = torch.zeros(1, device=dev)

    def loop(K):
        side.wait_stream(main)
        with torch.cuda.stream(side):
            sdm_fwd_phase1(bank, *fargs, workspace=ws_pair[0], chunk=wl.C, valid_tokens=t["valid"], stream=side)
            p1_done[0].record(side)
        for k in range(K):
            b = k % 2
            main.wait_event(p1_done[b])
            sdm_fwd_phase2(bank, *fargs, workspace=ws_pair[b], out=out, chunk=wl.C, valid_tokens=t["valid"],
                           stream=main)
            p2_done[b].record(main)
            if k + 1 < K:
                n = (k + 1) % 2
                with torch.cuda.stream(side):
                    if k >= 1:
                        side.wait_event(p2_done[n])
                    marker.add_(1.0)
                    sdm_fwd_phase1(bank, *fargs, workspace=ws_pair[n], chunk=wl.C, valid_tokens=t["valid"],
                                   stream=side)
                    p1_done[n].record(side)
        main.wait_stream(side)

    print(f"bench: timing {args.steps} overlapped steps", file=sys.stderr, flush=True)
    loop(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop(args.steps)
    torch.cuda.synchronize()
    return 1000.0 * (time.perf_counter() - t0) / args.steps


if __name__ == "__main__":
    main()
