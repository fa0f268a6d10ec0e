#!/usr/bin/env python3
"""Benchmark of batched draft-token verification on one MI355X.

Default workload: stochastic verification of B=64 requests with k=3 drafts over
a V=128256 bf16 vocabulary at temperature 0.8 (rank-Zipf synthetic logits,
seed 0).  One step is one full ``spec_verify_stochastic`` call (streaming
statistics + accept/reject + residual/bonus sampling) on inputs already resident
in device memory.  Inputs rotate over enough copies (>= 1 GiB in total) that the
256 MB last-level cache cannot serve a step from the previous one.

Prints ONE JSON line: throughput in verified rows/s (B * (k+1) per step); the
roofline of the call's dominant kernel (for the plain stochastic call, the
one-launch kernel that is the whole call), as algorithmic bytes (one read of each
logits tensor) over that kernel's own start/end event timestamps in a second run
of the timed steps, with the whole call's fraction beside it; and the CPU
oracle on the same workload (one host thread, then one thread per core), which
also reports how many of the step's requests it finds ambiguous and how many
differ from the GPU's.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "verified rows/sec (B·(k+1)) and achieved HBM GB/s at V=128256 bf16"
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="c3",
                    choices=["c1", "c2-greedy", "c2-stochastic", "c3", "c4", "c5", "c5-stochastic"])
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies to rotate over (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--top-k", type=int, default=0,
                    help="stochastic workloads: top-k filter of every row (0: off)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="stochastic workloads: top-p filter of every row (1: off)")
    ap.add_argument("--min-p", type=float, default=0.0,
                    help="stochastic workloads: min-p filter of every row (0: off)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--bare-read", action="store_true",
                    help="only time plain reads of the workload's logits bytes: the library's "
                         "argmax stream and torch's amax over the same bytes (the streaming "
                         "ceiling of this box)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph holding one call per input copy "
                         "(how a serving loop issues launch-bound calls) instead of eager calls")
    ap.add_argument("--pmc-summary", nargs=4, metavar="CSV",
                    help="write profiles/dominant_kernel_<workload>_pmc.json from four rocprofv3 "
                         "--pmc counter_collection.csv files: FETCH_SIZE and WRITE_SIZE of this "
                         "workload's run, then of a --copy-probe run (the calibration)")
    ap.add_argument("--pmc-kernel", default="sv::plain_kernel",
                    help="name fragment of the kernel the --pmc-summary figures are for")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the parallel oracle leg (0: the host's core count)")
    return ap.parse_args()


# The source file of each mode's timed kernel (with every shared header).
KERNEL_SOURCE = {"stochastic": "sv_stochastic.hip", "filtered": "sv_filter.hip",
                 "greedy": "sv_argmax.hip", "tree": "sv_argmax.hip",
                 "tree-stochastic": "sv_tree_stochastic.hip"}


def source_hash(kernel_file: str) -> str:
    """Hash of the timed kernel's source file and the shared headers: counters
    taken on other sources no longer describe it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_token_verification_verify_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == kernel_file or name.endswith(".hpp"):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def make_case(name: str, seed: int):
    from draft_token_verification_verify_amd import workloads as wl

    return {
        "c1": wl.c1, "c2-greedy": wl.c2_greedy, "c2-stochastic": wl.c2_stochastic,
        "c3": wl.c3, "c4": wl.c4, "c5": wl.c5,
        "c5-stochastic": lambda s: wl.stochastic_tree_case(
            s, 32, 60, 6, 128256, "bf16", target_sd=3.0, draft_noise_sd=1.0,
            name="c5-stochastic-tree-B32-N60-depth6-V128256-bf16"),
    }[name](seed)


def mode_of(case) -> str:
    from draft_token_verification_verify_amd import workloads as wl

    if isinstance(case, wl.StochasticCase):
        return "stochastic"
    if isinstance(case, wl.GreedyCase):
        return "greedy"
    if isinstance(case, wl.StochasticTreeCase):
        return "tree-stochastic"
    return "tree"


def device_inputs(case, copies: int):
    import numpy as np
    import torch

    from draft_token_verification_verify_amd.workloads import to_device as to_dev

    mode = mode_of(case)
    base = {"target": to_dev(case.target, case.dtype)}
    if mode == "stochastic":
        if case.k > 0:
            base["draft"] = to_dev(case.draft, case.dtype)
            base["draft_tokens"] = to_dev(case.draft_tokens.astype(np.int32))
        base["uniforms"] = to_dev(case.uniforms.astype(np.float32))
    elif mode == "greedy":
        base["draft_tokens"] = to_dev(case.draft_tokens.astype(np.int32))
    elif mode == "tree-stochastic":
        base["draft"] = to_dev(case.draft, case.dtype)
        base["node_tokens"] = to_dev(case.node_tokens.astype(np.int32))
        base["paths"] = to_dev(case.paths.astype(np.int32))
        base["uniforms"] = to_dev(case.uniforms.astype(np.float32))
    else:
        base["node_tokens"] = to_dev(case.node_tokens.astype(np.int32))
        base["paths"] = to_dev(case.paths.astype(np.int32))
    sets = [base]
    for _ in range(copies - 1):
        sets.append({k: v.clone() for k, v in base.items()})
    torch.cuda.synchronize()
    return sets


def make_step(case, sets, filt=None):
    """Return step(i) running one verification call on input copy i % len(sets)
    (the filtered stochastic call when ``filt`` = (top_k, top_p, min_p))."""
    import torch

    import draft_token_verification_verify_amd as sv

    mode = mode_of(case)
    dev = sets[0]["target"].device
    ws = sv.Workspace()
    if mode == "stochastic":
        out = torch.empty((case.B, case.k + 1), dtype=torch.int32, device=dev)
        acc = torch.empty((case.B,), dtype=torch.int32, device=dev)

        def step(i):
            s = sets[i % len(sets)]
            if filt is None:
                sv.spec_verify_stochastic(s["target"], s.get("draft"), s.get("draft_tokens"),
                                          s["uniforms"], case.temperature, out_tokens=out,
                                          num_accepted=acc, workspace=ws)
            else:
                sv.spec_verify_stochastic_filtered(s["target"], s.get("draft"),
                                                   s.get("draft_tokens"), s["uniforms"],
                                                   case.temperature, *filt, out_tokens=out,
                                                   num_accepted=acc, workspace=ws)
        return step, out, acc
    if mode == "greedy":
        out = torch.empty((case.B, case.k + 1), dtype=torch.int32, device=dev)
        acc = torch.empty((case.B,), dtype=torch.int32, device=dev)

        def step(i):
            s = sets[i % len(sets)]
            sv.spec_verify_greedy(s["target"], s["draft_tokens"], out_tokens=out,
                                  num_accepted=acc, workspace=ws)
        return step, out, acc
    if mode == "tree-stochastic":
        out = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)
        acc = torch.empty((case.B,), dtype=torch.int32, device=dev)
        nodes = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)

        def step(i):
            s = sets[i % len(sets)]
            sv.spec_verify_tree_stochastic(s["target"], s["draft"], s["node_tokens"], s["paths"],
                                           s["uniforms"], case.temperature, out_tokens=out,
                                           num_accepted=acc, accepted_nodes=nodes, workspace=ws,
                                           check=False)
        step.nodes = nodes
        return step, out, acc
    out = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)
    acc = torch.empty((case.B,), dtype=torch.int32, device=dev)
    best = torch.empty((case.B,), dtype=torch.int32, device=dev)
    nodes = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        sv.spec_verify_tree(s["target"], s["node_tokens"], s["paths"], out_tokens=out,
                            num_accepted=acc, best_path=best, accepted_nodes=nodes,
                            workspace=ws)
    return step, out, acc


def time_steps(step, steps: int, warmup: int) -> float:
    """Mean ms per step over `steps` calls, bracketed by synchronisations."""
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_steps_graph(step, steps: int, warmup: int, n_sets: int):
    """Mean ms per call over replays of a graph that holds n_sets consecutive
    calls (one per input copy), bracketed by synchronisations; and the number of
    calls timed.  Warm-up runs on the capture stream first, so that the library's
    workspace for that stream exists before the capture."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(warmup, 1)):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(n_sets):
            step(i)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // n_sets)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (reps * n_sets), reps * n_sets


def time_streaming_kernel(step, steps: int, warmup: int):
    """Per-launch durations (ms) of the streaming kernel over a second run of the
    same steps, in which the library attaches a start/stop event pair to each
    streaming-kernel launch (the kernel's own start and end timestamps, on the
    stream it runs on).  Attached events add a few microseconds between the
    kernels of a step, so the step rate comes from the plain run."""
    import torch

    from draft_token_verification_verify_amd import _lib

    lib = _lib.load()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for e in evs:  # materialise the underlying hipEvent_t handles
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    _lib.check("spec_verify_profile_events", lib.spec_verify_profile_events(handles, steps))
    try:
        for i in range(steps):
            step(warmup + i)
        torch.cuda.synchronize()
    finally:
        lib.spec_verify_profile_events(None, 0)
    return [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(steps)]


def streaming_bytes(case) -> int:
    """Algorithmic bytes of the streaming kernel: one read of every logits row."""
    if mode_of(case) == "stochastic":
        return case.target.nbytes + (case.draft.nbytes if case.k > 0 else 0)
    if mode_of(case) == "tree-stochastic":
        return case.target.nbytes + case.draft.nbytes
    return case.target.nbytes


def tree_walk_bytes(case, nodes, acc) -> int:
    """Algorithmic bytes of a stochastic tree walk: one read of the target row of
    every visited node (the root and the accepted nodes) and of the draft row of
    every visited node whose children were tested."""
    import numpy as np

    row = case.V * (2 if case.dtype == "bf16" else 4)
    total = 0
    for b in range(case.B):
        has_child = np.zeros(case.N + 1, bool)
        par = case.parents[b]
        has_child[par[par >= 0]] = True
        visited = [0] + [int(n) for n in nodes[b, :int(acc[b])]]
        for depth, n in enumerate(visited):
            total += row
            if has_child[n] and depth + 1 < case.L:
                total += row
    return total


WORKLOAD_MODE = {"c1": "stochastic", "c2-stochastic": "stochastic", "c3": "stochastic",
                 "c4": "stochastic", "c2-greedy": "greedy", "c5": "tree",
                 "c5-stochastic": "tree-stochastic"}


def pmc_summary(args):
    """HBM bytes per launch of one kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters (KiB per dispatch), each scaled by what the same counter reads for
    the plain 1 GiB device copy of --copy-probe (1 GiB read, 1 GiB written)."""
    import csv

    import numpy as np

    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.pmc_summary

    def values(path, counter, match):
        with open(path) as f:
            return [float(r["Counter_Value"]) for r in csv.DictReader(f)
                    if r["Counter_Name"] == counter and match(r["Kernel_Name"])]

    def kernel(name):
        return args.pmc_kernel in name

    def copy(name):
        return name.startswith("__amd_rocclr_copyBuffer")

    fetch = values(fetch_csv, "FETCH_SIZE", kernel)
    write = values(write_csv, "WRITE_SIZE", kernel)
    cf = values(cfetch_csv, "FETCH_SIZE", copy)
    cw = values(cwrite_csv, "WRITE_SIZE", copy)
    if not (fetch and write and cf and cw):
        raise SystemExit("pmc-summary: a counter file holds no dispatch of the kernel or the copy")
    # the 1 GiB copies (the probe's largest dispatches)
    cf = [v for v in cf if v >= 0.9 * max(cf)]
    cw = [v for v in cw if v >= 0.9 * max(cw)]
    kib = float(1 << 20)  # 1 GiB in KiB
    f_kib, w_kib = float(np.mean(fetch)), float(np.mean(write))
    ff, wf = kib / float(np.mean(cf)), kib / float(np.mean(cw))
    mode = WORKLOAD_MODE[args.workload]
    rec = {
        "workload": args.workload,
        "kernel": args.pmc_kernel,
        "source_hash": source_hash(KERNEL_SOURCE[mode]),
        "fetch_kib_per_dispatch": f_kib,
        "write_kib_per_dispatch": w_kib,
        "dispatches": [len(fetch), len(write)],
        "copy_probe": {"bytes": 1 << 30, "fetch_kib": float(np.mean(cf)),
                       "write_kib": float(np.mean(cw)), "fetch_factor": ff, "write_factor": wf},
        "hbm_read_bytes_per_launch": f_kib * ff * 1024.0,
        "hbm_write_bytes_per_launch": w_kib * wf * 1024.0,
        "hbm_bytes_per_launch": (f_kib * ff + w_kib * wf) * 1024.0,
    }
    path = os.path.join(PROFILES, f"dominant_kernel_{args.workload}_pmc.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec), flush=True)


def load_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"dominant_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_one(case, b, fkw):
    """The oracle on request b alone (one ctypes call: it releases the GIL)."""
    import oracle

    sl = slice(b, b + 1)
    mode = mode_of(case)
    if mode == "stochastic":
        return oracle.stochastic(case.target[sl], case.draft[sl] if case.k > 0 else None,
                                 case.draft_tokens[sl], case.uniforms[sl], case.temperature, **fkw)
    if mode == "greedy":
        return oracle.greedy(case.target[sl], case.draft_tokens[sl])
    if mode == "tree-stochastic":
        return oracle.tree_stochastic(case.target[sl], case.draft[sl], case.node_tokens[sl],
                                      case.paths[sl], case.uniforms[sl], case.temperature)
    return oracle.tree(case.target[sl], case.node_tokens[sl], case.paths[sl])


def cpu_baseline(case, seconds: float, gpu_out, gpu_acc, threads: int, filt=None):
    """The oracle (fp64 C, one request per call) on the same workload: one host
    thread for about `seconds`, then `threads` host threads (one request per
    call, calls in parallel) for about the same time.  The oracle's outputs on
    every request of the step are also compared with the GPU's (the stochastic
    modes count the requests the oracle finds ambiguous and those that differ)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    fkw = {} if filt is None else dict(top_k=filt[0], top_p=float(np.float32(filt[1])),
                                       min_p=float(np.float32(filt[2])))
    rows_per_req = case.rows // case.B
    # one thread
    done, times = 0, []
    t0 = time.perf_counter()
    while True:
        t1 = time.perf_counter()
        _oracle_one(case, done % case.B, fkw)
        times.append(time.perf_counter() - t1)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    single = done * rows_per_req / el
    # `threads` threads, about the same time
    n_par = max(threads * int(round(done / el * seconds / max(threads, 1))), threads)
    n_par = max(n_par, threads)
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda i: _oracle_one(case, i % case.B, fkw), range(n_par)))
        el_par = time.perf_counter() - t0
    parallel = n_par * rows_per_req / el_par
    out = dict(value=single, unit="rows/s", cores=1, kind="oracle",
               sample=f"{done} requests of {case.name} (seed {case.meta.get('seed')})"
                      f"{'' if filt is None else ' with filters ' + str(fkw)}, "
                      f"one request per call, {el:.1f} s on one host thread",
               per_request_ms_p10_p50_p90=[float(np.percentile(times, q)) * 1e3
                                           for q in (10, 50, 90)],
               parallel={"value": parallel, "unit": "rows/s", "cores": threads,
                         "sample": f"{n_par} requests, {threads} host threads (one request "
                                   f"per call), {el_par:.1f} s"},
               host_cpu=cpu_model(), host_threads_available=os.cpu_count())
    # parity over the step's requests (every request of the workload)
    mode = mode_of(case)
    if mode in ("stochastic", "tree-stochastic"):
        if mode == "stochastic":
            ref = oracle.stochastic(case.target, case.draft if case.k > 0 else None,
                                    case.draft_tokens, case.uniforms, case.temperature, **fkw)
            amb = oracle.ambiguous_requests(ref["margins"], 1e-6,
                                            ref.get("filter_margins") if filt else None, 1e-9)
        else:
            ref = oracle.tree_stochastic(case.target, case.draft, case.node_tokens, case.paths,
                                         case.uniforms, case.temperature)
            amb = oracle.ambiguous_requests(ref["margins"], 1e-6)
    elif mode == "greedy":
        ref = oracle.greedy(case.target, case.draft_tokens)
        amb = np.zeros(case.B, bool)
    else:
        ref = oracle.tree(case.target, case.node_tokens, case.paths)
        amb = np.zeros(case.B, bool)
    same = (gpu_acc == ref["num_accepted"]) & np.all(gpu_out == ref["out_tokens"], axis=1)
    out["parity"] = {"requests": int(case.B), "rows": int(case.rows),
                     "ambiguous_requests": int(amb.sum()),
                     "ambiguous_requests_differing": int((amb & ~same).sum()),
                     "non_ambiguous_requests_differing": int((~amb & ~same).sum()),
                     "guard_band": 1e-6}
    return out


def copy_probe():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def bare_read(args):
    """Plain reads of the workload's logits bytes, rotating over >= 1 GiB of
    copies like the timed workload: the library's argmax stream over every
    logits row (the tree call with no paths: one 16-byte-vector tile per
    (row, chunk) with a max and an index per element, then a one-workgroup-per-
    request epilogue), timed per call and, through the profiling hook, the
    streaming kernel alone; and torch's amax over the same bytes."""
    import numpy as np
    import torch

    import draft_token_verification_verify_amd as sv
    from draft_token_verification_verify_amd import _lib

    case = make_case(args.workload, args.seed)
    nbytes = streaming_bytes(case)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    esize = 2 if case.dtype == "bf16" else 4
    V = case.V
    rows = nbytes // (V * esize)
    B = case.B
    R = rows // B
    copies = max(1, math.ceil((1 << 30) / nbytes))
    bufs = [torch.randn(B, R, V, device="cuda").to(dt) for _ in range(copies)]
    nt = torch.zeros((B, R), dtype=torch.int32, device="cuda")
    paths = torch.zeros((B, 0, 1), dtype=torch.int32, device="cuda")
    ws = sv.Workspace()
    outs = [torch.empty((B, 1), dtype=torch.int32, device="cuda"),
            torch.empty((B,), dtype=torch.int32, device="cuda")]

    def stream(x):
        sv.spec_verify_tree(x, nt, paths, out_tokens=outs[0], num_accepted=outs[1], workspace=ws)

    res = {}
    for name, fn in (("argmax_stream_call", stream), ("torch_amax", lambda x: torch.amax(x, dim=2))):
        for i in range(args.warmup):
            fn(bufs[i % copies])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            evs[i][0].record()
            fn(bufs[i % copies])
            evs[i][1].record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        res[name] = {"us_median": float(np.median(us)), "us_p10": float(np.percentile(us, 10)),
                     "us_p90": float(np.percentile(us, 90)),
                     "gbps_median": nbytes / (np.median(us) * 1e-6) / 1e9}
    kms = time_streaming_kernel(lambda i: stream(bufs[i % copies]), args.steps, args.warmup)
    us = np.array(kms) * 1e3
    res["argmax_stream_kernel"] = {
        "us_median": float(np.median(us)), "us_p10": float(np.percentile(us, 10)),
        "us_p90": float(np.percentile(us, 90)),
        "gbps_median": nbytes / (np.median(us) * 1e-6) / 1e9}
    print(json.dumps({"bare_read_bytes": nbytes, "workload": case.name, "rows": int(rows),
                      "copies": copies, "peak_gbps": HBM_PEAK_GBPS, **res}), flush=True)
    del _lib


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: run it with --gpus 1 (requests would shard across "
              "GPUs with no exchange; no multi-GPU run is made here)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.bare_read:
        bare_read(args)
        return

    t_gen = time.perf_counter()
    case = make_case(args.workload, args.seed)
    print(f"bench: generated {case.name} in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    nbytes = streaming_bytes(case)
    copies = args.copies or max(1, math.ceil((1 << 30) / nbytes))
    if mode_of(case) == "tree-stochastic" and not args.copies:
        copies = 8  # a walk reads a few rows per request: rotate far beyond the MALL
    sets = device_inputs(case, copies)
    filt = None
    if mode_of(case) == "stochastic" and (0 < args.top_k < case.V or args.top_p < 1.0
                                          or args.min_p > 0.0):
        filt = (args.top_k, args.top_p, args.min_p)
    step, out, acc = make_step(case, sets, filt)
    print(f"bench: {copies} input copies, {args.warmup} warmup + {args.steps} timed steps",
          file=sys.stderr, flush=True)

    import draft_token_verification_verify_amd as sv
    from draft_token_verification_verify_amd import _lib

    timed_steps = args.steps
    if args.graph:
        ms, timed_steps = time_steps_graph(step, args.steps, args.warmup, copies)
    else:
        ms = time_steps(step, args.steps, args.warmup)
    # The dominant kernel of the timed call, timed on its own stream through the
    # library's profiling hook (a second run of the same steps).
    kernel_ms = time_streaming_kernel(step, args.steps, args.warmup)
    plain = mode_of(case) == "stochastic" and filt is None
    stats_pass = None
    if plain:
        # Beside it: the two-kernel schedule's first kernel (statistics and the
        # per-request decisions, the algorithmic read), for reference.
        sv.spec_verify_set_schedule(_lib.SCHEDULE_TWO_KERNELS)
        try:
            two_ms = time_streaming_kernel(step, args.steps, args.warmup)
        finally:
            sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)
        stats_pass = {
            "kernel": "sv::stats_kernel (two-kernel schedule: statistics only)",
            "us_mean": float(np.mean(two_ms)) * 1e3,
            "achieved_gbps": nbytes / (float(np.mean(two_ms)) * 1e-3) / 1e9,
        }
    k_avg = float(np.mean(kernel_ms))
    if mode_of(case) == "tree-stochastic":
        # the walk reads only the visited rows: the same outputs on every copy
        nbytes = tree_walk_bytes(case, step.nodes.cpu().numpy(), acc.cpu().numpy())
    rows = case.rows
    value = rows / (ms * 1e-3)
    achieved = nbytes / (k_avg * 1e-3) / 1e9
    n_acc = acc.cpu().numpy()
    src_hash = source_hash(KERNEL_SOURCE["filtered" if filt is not None else mode_of(case)])
    kname = ("filter selection kernel (filtered call)" if filt is not None else
             "one-launch kernel (statistics, decisions and sampling: the whole call)" if plain
             else "tree walk kernel (each request's walk split over workgroups)"
             if mode_of(case) == "tree-stochastic" else "argmax kernel")
    traffic = load_traffic(args.workload, src_hash) if filt is None else None
    wname = case.name if filt is None else (
        f"{case.name}-topk{args.top_k}-topp{args.top_p:g}-minp{args.min_p:g}")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": wname,
            "mode": mode_of(case),
            "B": case.B,
            "rows_per_step": rows,
            "V": case.V,
            "logits_bytes": nbytes,
            "input_copies": copies,
            "launch": "graph replay" if args.graph else "eager",
            "seed": args.seed,
            **({"k": case.k} if mode_of(case) in ("stochastic", "greedy")
               else {"N": case.N, "P": case.P, "L": case.L}),
            **({"temperature": case.temperature}
               if mode_of(case) in ("stochastic", "tree-stochastic") else {}),
            **({} if filt is None else {"top_k": args.top_k, "top_p": args.top_p,
                                        "min_p": args.min_p}),
        },
        "hbm_gbps_whole_call": nbytes / (ms * 1e-3) / 1e9,
        "whole_call_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel_us_mean": k_avg * 1e3,
            "kernel_us_p10_p50_p90": [float(np.percentile(kernel_ms, q)) * 1e3
                                      for q in (10, 50, 90)],
            "algorithmic_bytes_per_launch": nbytes,
            "source_hash": src_hash,
        },
        "statistics_pass": stats_pass,
        "num_accepted_histogram": np.bincount(n_acc, minlength=(rows // case.B)).tolist(),
        "acceptance_length": float(n_acc.mean() + 1.0),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        threads = args.cpu_threads or min(os.cpu_count() or 1, 16)
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, out.cpu().numpy(), n_acc,
                                            threads, filt)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
