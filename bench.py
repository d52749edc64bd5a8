"""Benchmark of the sparse MLA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the library (gather + QK^T + softmax + PV, plus the
split-K combine when the call splits) on one batch of synthetic input that is
already resident in HBM.  The default workload is the GLM-5.3-Flash-like bf16
decode: 32 sequences x 1 query token, 16 heads, 512-wide rope-free rows, top-k
2048 out of 131072-token paged contexts (block size 64).  Eight independent
index sets (and q) rotate from step to step so the 512 MiB they touch does
not fit the 256 MB Infinity Cache.

The K steps are captured once as a HIP graph and replayed BATCHES times, each
replay bracketed by synchronisations; the median replay gives the whole-job
rate (every replay's time is in `batch_ms`).  Before the timed replays the
graph is replayed untimed for about 0.1 s (besides the W warmup calls): the
clocks need that long to settle (20-call replays of the 576-wide workload ran
1.31 - 1.50 ms each right after set-up, ~1.15 ms once settled).

Prints ONE JSON line: value = gathered KV bytes / second (whole job), plus
`roofline` for the main kernel (algorithmic gathered bytes / its own average
duration, timed with HIP events the library records around it on the same
stream; `frac_call` the same bytes over the whole call; `frac_measured` and
`frac_call_measured` against the gather-only ceiling of the same index stream)
and `cpu_baseline` (the fp64 oracle on the host, same workload).  The default
run also measures the device ceilings (`ceilings`: streaming read, gather-only
on each workload's own index stream, bf16 / e4m3 MFMA loops, from
libsmla_ceiling.so) and times the other workloads the same way (`workloads`:
e4m3 decode, the largest prefill shape, 576-wide rows with 128 heads in bf16 and
e4m3), each with its own roofline fractions.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
INDEX_SETS = 8
BATCHES = 5


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="split count passed to the library (0 = its own choice; a sensitivity "
                         "setting, not the workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, run --steps plain device copies of BYTES "
                         "(fp32 x * 1 into another buffer): the reference for scaling the HBM "
                         "byte counters of rocprofv3")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("KERNEL_FETCH", "KERNEL_WRITE",
                                                           "COPY_FETCH", "COPY_WRITE"),
                    help="instead of the benchmark, turn four rocprofv3 --pmc output folders "
                         "(FETCH_SIZE / WRITE_SIZE of this workload, then of --copy-calibration "
                         "--copy-bytes) into profiles/traffic_<workload>.json")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the device-ceiling probes (stream read, gather-only, MFMA loops)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the device ceilings (streaming read, MFMA loops, gather-only on "
                         "every decode workload's index stream) and print them")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only --workload (the default run also times the other workloads)")
    ap.add_argument("--sensitivity", action="store_true",
                    help="also time (not part of value): each call after a 1 GiB read that "
                         "evicts the caches (cold; for prefill this is the cold first call), "
                         "the same workload with every top-k list sorted by slot, and with "
                         "block size 1 (every position its own randomly placed slot)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t pairs via the HIP runtime (the library records them on its stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def pair(self, i):
        return self.ev[2 * i], self.ev[2 * i + 1]

    def elapsed_ms(self, i) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[2 * i], self.ev[2 * i + 1]) == 0
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


# the sources of the forward pass's kernels and their launch configuration; the
# fused RoPE / cache write is a kernel of its own and does not enter the hash
FWD_SOURCES = ("smla_api.hip", "smla_common.h", "smla_device.h", "smla_kernels.h", "smla_kernels.hip",
               "smla_prefill.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mla_attention_03_amd", "csrc")
    for f in FWD_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, launches_bytes: float):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int, steps: int) -> None:
    """A plain streaming copy of known size: its FETCH_SIZE / WRITE_SIZE per
    dispatch give the factor from counter units to HBM bytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                      "launches": max(steps, 1)}), flush=True)


def _counter_per_dispatch(folder: str, counter: str, select):
    """Mean over dispatches of `counter` (summed over its instances) for the
    kernels whose name passes `select`, from a rocprofv3 --pmc csv folder."""
    import collections
    import csv
    import glob
    per = collections.defaultdict(float)
    names = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter or not select(row["Kernel_Name"]):
                continue
            per[row["Dispatch_Id"]] += float(row["Counter_Value"])
            names[row["Dispatch_Id"]] = row["Kernel_Name"]
    if not per:
        raise RuntimeError(f"no {counter} rows in {folder}")
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals), sorted(set(names.values()))


def traffic_summary(workload: str, dirs, copy_bytes: int) -> None:
    kf, kw, cf, cw = dirs
    main = lambda k: "smla_" in k and "combine" not in k and "quantize" not in k
    big = lambda k: "MulFunctor" in k           # the x * 1 copy, not the fill before it
    fetch, n_f, names = _counter_per_dispatch(kf, "FETCH_SIZE", main)
    write, n_w, _ = _counter_per_dispatch(kw, "WRITE_SIZE", main)
    c_fetch, _, c_names = _counter_per_dispatch(cf, "FETCH_SIZE", big)
    c_write, _, _ = _counter_per_dispatch(cw, "WRITE_SIZE", big)
    f_scale = copy_bytes / c_fetch      # HBM bytes per counter unit, reads
    w_scale = copy_bytes / c_write      # ... writes
    rec = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "kernels": names, "dispatches": [n_f, n_w],
           "fetch_size_per_dispatch": round(fetch, 1), "write_size_per_dispatch": round(write, 1),
           "copy_kernel": c_names, "copy_bytes": copy_bytes,
           "copy_fetch_size": round(c_fetch, 1), "copy_write_size": round(c_write, 1),
           "read_bytes_per_unit": round(f_scale, 3), "write_bytes_per_unit": round(w_scale, 3),
           "hbm_read_bytes_per_launch": int(fetch * f_scale),
           "hbm_write_bytes_per_launch": int(write * w_scale),
           "hbm_bytes_per_launch": int(fetch * f_scale + write * w_scale)}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec), flush=True)


WARM_S = 0.1   # untimed graph replays before timing: the clocks settle after ~100 ms of work


def warm_replays(graph) -> None:
    """Replay `graph` untimed for about WARM_S seconds (at least 3 times)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < WARM_S:
        graph.replay()
        torch.cuda.synchronize()
        n += 1


def graph_us_per_call(call, steps: int) -> float:
    """Median over BATCHES graph replays of `steps` captured calls, per call."""
    import numpy as np
    import torch
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(steps):
            call(i)
    warm_replays(graph)
    ms = []
    for _ in range(BATCHES):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        ms.append(t0.elapsed_time(t1))
    del graph
    return float(np.median(ms)) / steps * 1e3


def sensitivity(spec, cases, call_case, steps: int) -> dict:
    """Timings that are not the workload (reported beside it): cold caches, lists
    sorted by slot, block size 1."""
    import dataclasses

    import numpy as np
    import torch

    from sparse_mla_attention_03_amd import synth
    res = {}
    # cold: a 1 GiB read between calls evicts L2 and the 256 MB Infinity Cache
    # (a read, so the caches hold clean lines: a write would leave dirty ones
    # whose write-back the call would pay for); only the call is timed (events
    # on the current stream, eager calls)
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    sink = torch.empty((), dtype=torch.float32, device="cuda:0")
    times = []
    for i in range(20):
        torch.sum(scratch, dim=0, out=sink)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        call_case(cases[i % len(cases)])
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1) * 1e3)
    res["cold_first_call_us"] = round(times[0], 3)
    res["cold_us_median"] = round(float(np.median(times)), 3)
    del scratch
    # every list sorted by slot (padding first): same rows, better locality
    srt = []
    for c in cases:
        idx = torch.sort(c.topk_idx, dim=1).values.contiguous()
        srt.append(dataclasses.replace(c, topk_idx=idx))
    res["sorted_lists_us"] = round(graph_us_per_call(lambda i: call_case(srt[i % len(srt)]), steps), 3)
    del srt
    # block size 1: every logical position is its own randomly placed slot
    spec1 = dataclasses.replace(spec, block_size=1)
    c1 = synth.make_case(spec1, device="cuda:0", index_sets=len(cases))
    c1 = c1 if isinstance(c1, list) else [c1]
    res["block_size_1_us"] = round(graph_us_per_call(lambda i: call_case(c1[i % len(c1)]), steps), 3)
    del c1
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cases, budget_s: float):
    """The fp64 oracle (as it stands) on the host: whole decode calls of the same
    workload, repeated over index sets until about `budget_s` seconds."""
    import numpy as np
    import oracle
    from tests.helpers import bits16, codes8

    done_bytes, t_total, n_calls, n_tok = 0, 0.0, 0, 0
    # stage host copies first (not timed): the rows each call gathers, remapped
    staged = []
    for case in cases:
        idx = case.topk_idx.cpu().numpy()
        N = case.kv_pool.shape[0] * case.kv_pool.shape[1]
        valid = (idx >= 0) & (idx < N)
        rows = np.unique(idx[valid]).astype(np.int64)
        remap = np.full(idx.shape, -1, np.int32)
        remap[valid] = np.searchsorted(rows, idx[valid])
        import torch
        flat = case.kv_pool.reshape(-1, case.kv_pool.shape[-1])
        sub = flat[torch.from_numpy(rows).to(flat.device)].cpu()
        kv = bits16(sub) if sub.dtype == torch.bfloat16 else codes8(sub)
        staged.append((bits16(case.q.cpu()), np.ascontiguousarray(kv), remap,
                       int(valid.sum()) * case.spec.Dqk * (2 if case.spec.kv_dtype == "bf16" else 1),
                       case))
        if len(staged) >= 2:
            break
    while t_total < budget_s and n_calls < 96:
        q, kv, remap, nbytes, case = staged[n_calls % len(staged)]
        t0 = time.perf_counter()
        oracle.sparse_mla_fwd(q, kv, remap, case.sm_scale, case.kv_scale)
        t_total += time.perf_counter() - t0
        done_bytes += nbytes
        n_calls += 1
        n_tok += q.shape[0]
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n_calls} whole calls of the same workload ({n_tok} query tokens, "
                      f"fp64 C oracle, OpenMP over (token, head)), {t_total:.1f} s",
            "us_per_call": round(t_total / n_calls * 1e6, 1)}, staged


def cpu_single_thread(staged) -> dict:
    """The same oracle on one host thread: one whole call of the workload."""
    import oracle
    threads = oracle.num_threads()
    q, kv, remap, nbytes, case = staged[0]
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.sparse_mla_fwd(q, kv, remap, case.sm_scale, case.kv_scale)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(nbytes / dt / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "one whole call of the same workload on one thread", "us_per_call": round(dt * 1e6, 1)}


# The fused q-RoPE / q-concat / KV-concat / cache write (the step in front of the
# forward pass), e4m3 q and cache: a decode batch of the 128-head RoPE model and
# one 8192-token sequence of the 16-head model.  (tokens, heads, cache slots)
ROPE_CACHE_WORKLOADS = {"rope_cache_decode": (64, 128, 64 * 32768),
                        "rope_cache_prefill": (8192, 16, 8192)}


def rope_cache_bench(args) -> None:
    """One JSON line: bytes the fused op must move per call (inputs read once,
    outputs written once) / time, against the HBM peak."""
    import numpy as np
    import torch

    from sparse_mla_attention_03_amd import synth
    from sparse_mla_attention_03_amd.binding import sparse_mla_rope_concat_cache

    T, H, N = ROPE_CACHE_WORKLOADS[args.workload]
    bs = 64
    case = synth.make_rope_case(T, H, N // bs, bs, max_pos=32768, seed=6)
    dev = torch.device("cuda:0")
    g = [t.to(dev) for t in (case.ql_nope, case.q_pe, case.kv_c, case.k_pe, case.positions,
                             case.cos_sin, case.slot_mapping)]
    cache = torch.zeros((N // bs, bs, 576), dtype=torch.uint8, device=dev)
    q_out = torch.empty((T, H, 576), dtype=torch.uint8, device=dev)

    def call():
        sparse_mla_rope_concat_cache(*g[:6], True, g[6], cache, q_out=q_out, q_fp8=True,
                                     q_scale=0.02, kv_scale=0.011)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            call()
    warm_replays(graph)
    batch_ms = []
    for _ in range(BATCHES):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        batch_ms.append(t0.elapsed_time(t1))
    ms = float(np.median(batch_ms)) / args.steps
    # per token: ql_nope and q_pe (bf16), kv_c and k_pe (bf16), cos/sin row (fp32),
    # position and slot (int64) read; q_out and the cache row (e4m3) written
    per_tok = H * (512 + 64) * 2 + (512 + 64) * 2 + 64 * 4 + 16 + H * 576 + 576
    gbs = T * per_tok / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "fused q-RoPE + q-concat + KV-cache write, algorithmic GB/s (1 MI355X)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "heads": H, "bytes_per_call": T * per_tok},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "batch_ms": [round(b, 4) for b in batch_ms]}), flush=True)


# Mixed batches: decode tokens with full top-2048 lists next to short lists
# (64 .. 512 entries), one call; every token has its own paged context.
# (heads, Dqk, context per token, decode tokens, short tokens)
MIXED_WORKLOADS = {"mixed_bf16": (16, 512, 16384, 32, 480),
                   "mixed_rope_bf16": (128, 576, 32768, 16, 112)}


def _graph_us(fn, steps, warmup):
    """Median of BATCHES graph replays of `steps` calls, in microseconds per call."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fn()
    warm_replays(graph)
    ms = []
    for _ in range(BATCHES):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        ms.append(t0.elapsed_time(t1))
    return float(np.median(ms)) / steps * 1e3, ms


def mixed_bench(args) -> None:
    """One JSON line: the per-token-length call on a mixed batch (gathered bytes of the
    valid entries / time), with the same batch as one padded call beside it."""
    import numpy as np
    import torch

    from sparse_mla_attention_03_amd import synth
    from sparse_mla_attention_03_amd.binding import (sparse_mla_fwd_ex, sparse_mla_fwd_varlen,
                                                     sparse_mla_workspace_bytes,
                                                     sparse_mla_workspace_bytes_varlen)

    H, D, ctx, Td, Ts = MIXED_WORKLOADS[args.workload]
    T, K = Td + Ts, 2048
    spec = synth.small_spec(T=T, H=H, Dqk=D, K=K, ctx=ctx, mode="decode", seed=8,
                            sm_scale=1.0 / np.sqrt(D))
    case = synth.make_case(spec, device="cuda:0")
    rng = np.random.default_rng(8)
    lens = np.concatenate([np.full(Td, K), rng.integers(64, 513, Ts)]).astype(np.int32)
    idx = case.topk_idx.cpu().numpy().copy()
    for t in range(T):
        idx[t, lens[t]:] = -1
    dev = torch.device("cuda:0")
    idx_d, lens_d = torch.from_numpy(idx).to(dev), torch.from_numpy(lens).to(dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws_p = torch.empty(max(sparse_mla_workspace_bytes(T, H, K, D, 0, 0), 16), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(sparse_mla_workspace_bytes_varlen(T, H, K, D, 0), dtype=torch.uint8, device=dev)
    us_v, batch_ms = _graph_us(lambda: sparse_mla_fwd_varlen(case.q, case.kv_pool, idx_d, lens_d, case.sm_scale,
                                                              out=out, lse=lse, workspace=ws_v),
                               args.steps, args.warmup)
    us_p, _ = _graph_us(lambda: sparse_mla_fwd_ex(case.q, case.kv_pool, idx_d, case.sm_scale, out=out, lse=lse,
                                                  workspace=ws_p), args.steps, args.warmup)
    nbytes = int(lens.sum()) * D * 2
    gbs = nbytes / (us_v * 1e-6) / 1e9
    print(json.dumps({
        "metric": "sparse-MLA mixed-batch gathered-KV HBM GB/s, per-token lengths (1 MI355X)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_v / 1e3, 6), "us_per_call": round(us_v, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "heads": H, "dqk": D, "decode_tokens": Td, "short_tokens": Ts,
                   "topk": K, "valid_entries": int(lens.sum()), "gathered_bytes_per_call": nbytes,
                   "padded_call_us": round(us_p, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "batch_ms": [round(b, 4) for b in batch_ms]}), flush=True)


# Workloads timed beside the headline one in the default run (every config of the
# benchmark table that fits one GPU; the prefill shape is the largest of the twelve)
SIDE_WORKLOADS = ("decode_fp8", "prefill_bf16_T2048_K2048", "rope_decode_bf16", "rope_decode_fp8")


class Ceilings:
    """The device's measured ceilings (libsmla_ceiling.so): streaming read, a
    gather of each workload's own index stream with no arithmetic, MFMA loops."""

    def __init__(self):
        import torch
        lib_path = os.path.join(ROOT, "sparse_mla_attention_03_amd", "csrc", "libsmla_ceiling.so")
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built (run __graft_entry__.build())")
        self.lib = ctypes.CDLL(lib_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        self.lib.smla_ceiling_stream_read.argtypes = [vp, i64, vp, i64, vp]
        self.lib.smla_ceiling_gather.argtypes = [vp, i64, i32, vp, i64, i32, i32, vp, i64, vp]
        self.lib.smla_ceiling_mfma.argtypes = [i32, i32, i32, vp, i64, vp]
        self.lib.smla_ceiling_lds_read.argtypes = [i32, i32, i32, vp, i64, vp]
        self.sink = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0")
        self.stream = torch.cuda.current_stream().cuda_stream

    def _time_ms(self, launch, reps: int) -> float:
        """Time per launch: `reps` launches captured as one HIP graph, median of
        BATCHES replays (as the workloads are timed: an isolated launch starts its
        workgroups on the eight XCDs microseconds apart, a replayed one does not)."""
        import numpy as np
        import torch
        launch(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.stream = side.cuda_stream
            launch(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            self.stream = torch.cuda.current_stream().cuda_stream
            for i in range(reps):
                launch(i)
        self.stream = torch.cuda.current_stream().cuda_stream
        warm_replays(graph)
        ts = []
        for _ in range(BATCHES):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record()
            graph.replay()
            t1.record()
            torch.cuda.synchronize()
            ts.append(t0.elapsed_time(t1) / reps)
        del graph
        return float(np.median(ts))

    def stream_read_gbs(self, nbytes: int = 2 << 30) -> float:
        import torch
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        def launch(_):
            assert self.lib.smla_ceiling_stream_read(buf.data_ptr(), nbytes, self.sink.data_ptr(),
                                                     self.sink.numel(), self.stream) == 0
        ms = self._time_ms(launch, 10)
        del buf
        torch.cuda.empty_cache()
        return nbytes / (ms * 1e-3) / 1e9

    PATTERNS = ("row, 8 in flight", "row, 16 in flight", "8 rows x 128 B, 8 in flight",
                "8 rows x 128 B, 16 in flight")

    def gather_gbs(self, cases, row_bytes: int) -> dict:
        """Best rate over access patterns and wave counts, rotating the workload's
        index sets; every combination is in `all`."""
        pool = cases[0].kv_pool
        N = pool.shape[0] * pool.shape[1]
        valid = sum(int(((c.topk_idx >= 0) & (c.topk_idx < N)).sum().item()) for c in cases) / len(cases)
        best, every = None, {}
        for pattern in range(4):
            for waves in (1024, 2048, 4096):
                def launch(i):
                    idx = cases[i % len(cases)].topk_idx
                    assert self.lib.smla_ceiling_gather(pool.data_ptr(), N, row_bytes, idx.data_ptr(), idx.numel(),
                                                        waves, pattern, self.sink.data_ptr(), self.sink.numel(),
                                                        self.stream) == 0
                ms = self._time_ms(launch, 2 * len(cases))
                gbs = valid * row_bytes / (ms * 1e-3) / 1e9
                every[f"{self.PATTERNS[pattern]}, {waves} waves"] = round(gbs, 1)
                if best is None or gbs > best["GB/s"]:
                    best = {"GB/s": round(gbs, 1), "us": round(ms * 1e3, 3), "waves": waves,
                            "pattern": self.PATTERNS[pattern]}
        best["all"] = every
        return best

    def lds_read_bytes_per_clk(self, waves_per_cu: int, clk_ghz: float = 2.4) -> float:
        """LDS read bandwidth per compute unit (bytes per clock at clk_ghz), one
        workgroup of waves_per_cu waves on each of 256 compute units."""
        blocks, iters = 256, 4000
        threads = 64 * waves_per_cu
        def launch(_):
            assert self.lib.smla_ceiling_lds_read(blocks, threads, iters, self.sink.data_ptr(),
                                                  self.sink.numel(), self.stream) == 0
        ms = self._time_ms(launch, 5)
        per_cu = threads * iters * 128 / (ms * 1e-3)
        return per_cu / (clk_ghz * 1e9)

    def mfma_tflops(self, fp8: bool) -> float:
        blocks, iters = 256 * 8, 2000
        def launch(_):
            assert self.lib.smla_ceiling_mfma(int(fp8), blocks, iters, self.sink.data_ptr(), self.sink.numel(),
                                              self.stream) == 0
        ms = self._time_ms(launch, 5)
        flop = blocks * 4 * iters * 8 * (65536 if fp8 else 16384)
        return flop / (ms * 1e-3) / 1e12


def measure_workload(name: str, steps: int, warmup: int, ceilings=None, keep_cases: bool = False,
                     num_splits: int = 0) -> dict:
    """Time one workload: whole calls (graph replays) and the main kernel alone
    (HIP events the library records around its own dispatch)."""
    import numpy as np
    import torch

    from sparse_mla_attention_03_amd import synth
    from sparse_mla_attention_03_amd.binding import (sparse_mla_fwd_ex, sparse_mla_num_splits,
                                                     sparse_mla_workspace_bytes)

    dev = torch.device("cuda:0")
    spec = synth.CONFIGS[name]
    cases = synth.make_case(spec, device="cuda:0", index_sets=INDEX_SETS)
    kvd = 0 if spec.kv_dtype == "bf16" else 1
    elem = 2 if spec.kv_dtype == "bf16" else 1
    S = sparse_mla_num_splits(spec.T, spec.H, spec.K, spec.Dqk, kvd, num_splits)
    ws_bytes = sparse_mla_workspace_bytes(spec.T, spec.H, spec.K, spec.Dqk, kvd, num_splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((spec.T, spec.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((spec.T, spec.H), dtype=torch.float32, device=dev)
    valid_rows = [int(((c.topk_idx >= 0) & (c.topk_idx < spec.N)).sum().item()) for c in cases]
    gathered = [v * spec.Dqk * elem for v in valid_rows]            # algorithmic bytes per call
    flops = [v * 2 * spec.H * (spec.Dqk + 512) for v in valid_rows]  # algorithmic FLOP per call

    def call(i, events=None):
        c = cases[i % INDEX_SETS]
        sparse_mla_fwd_ex(c.q, c.kv_pool, c.topk_idx, c.sm_scale, c.kv_scale, out=out, lse=lse,
                          workspace=ws, num_splits=num_splits, kernel_events=events)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # ---- whole-job timing: the K calls captured once as a HIP graph (no host
    # launch overhead inside the timed region), replayed back to back
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(steps):
            call(i)
    graph.replay()
    torch.cuda.synchronize()
    # a replay must reproduce the eager result of its last call bit for bit
    g_out, g_lse = out.clone(), lse.clone()
    call(steps - 1)
    torch.cuda.synchronize()
    if not (torch.equal(g_out.view(torch.int16), out.view(torch.int16)) and torch.equal(g_lse, lse)):
        raise RuntimeError(f"{name}: graph replay differs from the eager call")
    warm_replays(graph)   # untimed: the clocks settle before the timed replays
    # BATCHES replays of the K calls, each bracketed by synchronisations; the
    # median batch is reported (all of them go into the line)
    batch_ms = []
    wall = 0.0
    for _ in range(BATCHES):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        wall += time.perf_counter() - wall0
        batch_ms.append(t0.elapsed_time(t1))
    del graph
    ms_total = float(np.median(batch_ms))
    ms_per_step = ms_total / steps
    bytes_total = sum(gathered[i % INDEX_SETS] for i in range(steps))
    flop_total = sum(flops[i % INDEX_SETS] for i in range(steps))
    avg_bytes, avg_flop = bytes_total / steps, flop_total / steps
    decode = spec.mode != "prefill"

    # ---- main-kernel timing: HIP events the library records around that kernel
    ev = HipEvents(steps)
    for i in range(steps):
        call(i, events=ev.pair(i))
    torch.cuda.synchronize()
    kern_ms = [ev.elapsed_ms(i) for i in range(steps)]
    ev.close()
    kern_avg_ms = float(np.mean(kern_ms))
    gbs_kernel = avg_bytes / (kern_avg_ms * 1e-3) / 1e9
    gbs_call = avg_bytes / (ms_per_step * 1e-3) / 1e9
    tf_kernel = avg_flop / (kern_avg_ms * 1e-3) / 1e12
    tf_call = avg_flop / (ms_per_step * 1e-3) / 1e12
    mfma_peak = BF16_PEAK_TFLOPS
    res = {"workload": name, "spec": spec, "splits": S, "us_per_call": round(ms_per_step * 1e3, 3),
           "main_kernel_us": round(kern_avg_ms * 1e3, 3), "gathered_bytes_per_call": int(avg_bytes),
           "flop_per_call": int(avg_flop), "gbs_call": round(gbs_call, 1), "gbs_kernel": round(gbs_kernel, 1),
           "tflops_call": round(tf_call, 2), "tflops_kernel": round(tf_kernel, 2),
           "batch_ms": [round(b, 4) for b in batch_ms], "wall_s": round(wall, 3)}
    if decode:
        res["value"], res["unit"] = round(bytes_total / (ms_total * 1e-3) / 1e9, 3), "GB/s"
        res["roofline"] = {"bound": "hbm", "achieved": round(gbs_kernel, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(gbs_kernel / HBM_PEAK_GBS, 4),
                           "frac_call": round(gbs_call / HBM_PEAK_GBS, 4),
                           "traffic": traffic_from_profiles(name, avg_bytes)}
        if ceilings is not None:
            g = ceilings.gather_gbs(cases, spec.Dqk * elem)
            res["gather_ceiling"] = g
            res["roofline"]["measured_peak"] = g["GB/s"]
            res["roofline"]["frac_measured"] = round(gbs_kernel / g["GB/s"], 4)
            res["roofline"]["frac_call_measured"] = round(gbs_call / g["GB/s"], 4)
    else:
        res["value"], res["unit"] = round(flop_total / (ms_total * 1e-3) / 1e12, 3), "TFLOP/s"
        res["roofline"] = {"bound": "mfma", "achieved": round(tf_kernel, 2), "peak": mfma_peak,
                           "unit": "TFLOP/s", "frac": round(tf_kernel / mfma_peak, 4),
                           "frac_call": round(tf_call / mfma_peak, 4),
                           "traffic": traffic_from_profiles(name, avg_bytes)}
        if ceilings is not None and getattr(ceilings, "mfma_bf16", None):
            res["roofline"]["measured_peak"] = round(ceilings.mfma_bf16, 1)
            res["roofline"]["frac_measured"] = round(tf_kernel / ceilings.mfma_bf16, 4)
    if spec.kv_dtype == "fp8" and spec.H >= 64:
        # at the ridge: the matrix side as well (e4m3 QK + bf16 PV)
        res["mfma_tflops_kernel"] = round(tf_kernel, 2)
    if keep_cases:
        res["_cases"] = cases
    else:
        del cases
        torch.cuda.empty_cache()
    return res


def _side_summary(r: dict) -> dict:
    keep = ("splits", "us_per_call", "main_kernel_us", "value", "unit", "gbs_call", "gbs_kernel",
            "tflops_call", "tflops_kernel", "roofline", "gather_ceiling", "batch_ms")
    return {k: r[k] for k in keep if k in r}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(args.workload, args.traffic_summary, args.copy_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sparse MLA "
              f"forward pass here runs on a single MI355X with no sharding or collectives.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.workload in ROPE_CACHE_WORKLOADS:
        rope_cache_bench(args)
        return
    if args.workload in MIXED_WORKLOADS:
        mixed_bench(args)
        return

    import torch

    from sparse_mla_attention_03_amd.binding import load_library, sparse_mla_fwd_ex

    load_library()
    ceil = None
    ceilings_line = None
    if not args.no_ceilings:
        ceil = Ceilings()
        ceil.mfma_bf16 = ceil.mfma_tflops(False)
        ceilings_line = {"stream_read_GBs": round(ceil.stream_read_gbs(), 1),
                         "mfma_bf16_TFLOPs": round(ceil.mfma_bf16, 1),
                         "mfma_fp8_TFLOPs": round(ceil.mfma_tflops(True), 1),
                         "lds_read_B_per_clk_per_cu_at_2.4GHz": {
                             f"{w} waves": round(ceil.lds_read_bytes_per_clk(w), 1) for w in (4, 8, 16)},
                         "gather_GBs": {}}
    if args.ceilings:
        from sparse_mla_attention_03_amd import synth
        for w in ("decode_bf16",) + SIDE_WORKLOADS:
            spec = synth.CONFIGS[w]
            if spec.mode == "prefill":
                continue
            cases = synth.make_case(spec, device="cuda:0", index_sets=INDEX_SETS)
            ceilings_line["gather_GBs"][w] = ceil.gather_gbs(cases, spec.Dqk * (2 if spec.kv_dtype == "bf16" else 1))
            del cases
            torch.cuda.empty_cache()
        print(json.dumps({"ceilings": ceilings_line}), flush=True)
        return

    main_res = measure_workload(args.workload, args.steps, args.warmup, ceil, keep_cases=True,
                                num_splits=args.num_splits)
    cases = main_res.pop("_cases")
    spec = main_res["spec"]
    if ceilings_line is not None and "gather_ceiling" in main_res:
        ceilings_line["gather_GBs"][args.workload] = main_res["gather_ceiling"]

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu, staged = cpu_baseline(cases, args.cpu_seconds)
        cpu1 = cpu_single_thread(staged)
    sens = None
    if args.sensitivity:
        out = torch.empty((spec.T, spec.H, 512), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.empty((spec.T, spec.H), dtype=torch.float32, device="cuda:0")

        def call_case(c):
            sparse_mla_fwd_ex(c.q, c.kv_pool, c.topk_idx, c.sm_scale, c.kv_scale, out=out, lse=lse,
                              num_splits=0)
        sens = sensitivity(spec, cases, call_case, args.steps)
    del cases
    torch.cuda.empty_cache()

    side = {}
    if not args.no_workloads and args.workload == "decode_bf16":
        for w in SIDE_WORKLOADS:
            r = measure_workload(w, args.steps, args.warmup, ceil)
            side[w] = _side_summary(r)
            if ceilings_line is not None and "gather_ceiling" in r:
                ceilings_line["gather_GBs"][w] = r["gather_ceiling"]

    line = {
        "metric": "sparse-MLA decode \u00b5s/call + gathered-KV HBM GB/s; prefill TFLOP/s (1 MI355X)",
        "value": main_res["value"],
        "unit": main_res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["us_per_call"] / 1e3, 6),
        "us_per_call": main_res["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.kv_dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "tokens": spec.T, "heads": spec.H, "dqk": spec.Dqk,
                   "dv": 512, "topk": spec.K, "context": spec.ctx, "block_size": spec.block_size,
                   "kv": spec.kv_dtype, "splits": main_res["splits"], "index_sets": INDEX_SETS,
                   "gathered_bytes_per_call": main_res["gathered_bytes_per_call"],
                   "tflops": main_res["tflops_call"]},
        "roofline": main_res["roofline"],
        "main_kernel_us": main_res["main_kernel_us"],
        "cpu_baseline": cpu,
        "cpu_baseline_1_thread": cpu1,
        "batch_ms": main_res["batch_ms"],
        "wall_s": main_res["wall_s"],
    }
    if ceilings_line is not None:
        line["ceilings"] = ceilings_line
    if side:
        line["workloads"] = side
    if sens is not None:
        line["sensitivity"] = sens
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
