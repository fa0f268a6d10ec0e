#!/usr/bin/env python3
"""Benchmark of batched draft-token verification on one MI355X.

Default workload: stochastic verification of B=64 requests with k=3 drafts over
a V=128256 bf16 vocabulary at temperature 0.8 (rank-Zipf synthetic logits,
seed 0).  One step is one full ``spec_verify_stochastic`` call (streaming
statistics + accept/reject + residual/bonus sampling) on inputs already resident
in device memory.  Inputs rotate over enough copies (>= 1 GiB in total) that the
256 MB last-level cache cannot serve a step from the previous one.

Prints ONE JSON line: throughput in verified rows/s (B * (k+1) per step), the
roofline of the streaming kernel (algorithmic bytes = one read of each logits
tensor, over that kernel's own start/end event timestamps in a second run of the
timed steps), and the CPU oracle's rate on a bounded sample of the same
workload.
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
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_token_verification_verify_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
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
                                           num_accepted=acc, accepted_nodes=nodes, workspace=ws)
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


def load_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"streaming_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(case, seconds: float, filt=None):
    """The oracle (single-threaded fp64 C) on whole requests of the same workload
    until about `seconds` of CPU time has been spent."""
    import numpy as np

    import oracle

    fkw = {} if filt is None else dict(top_k=filt[0], top_p=float(np.float32(filt[1])),
                                       min_p=float(np.float32(filt[2])))
    mode = mode_of(case)
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % case.B
        sl = slice(b, b + 1)
        if mode == "stochastic":
            oracle.stochastic(case.target[sl], case.draft[sl] if case.k > 0 else None,
                              case.draft_tokens[sl], case.uniforms[sl], case.temperature, **fkw)
        elif mode == "greedy":
            oracle.greedy(case.target[sl], case.draft_tokens[sl])
        elif mode == "tree-stochastic":
            oracle.tree_stochastic(case.target[sl], case.draft[sl], case.node_tokens[sl],
                                   case.paths[sl], case.uniforms[sl], case.temperature)
        else:
            oracle.tree(case.target[sl], case.node_tokens[sl], case.paths[sl])
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    rows_per_req = case.rows // case.B
    return dict(value=done * rows_per_req / el, unit="rows/s", cores=1, kind="oracle",
                sample=f"{done} requests of {case.name} (seed {case.meta.get('seed')})"
                       f"{'' if filt is None else ' with filters ' + str(fkw)}, "
                       f"one request per call, {el:.1f} s on one host thread")


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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: run it with --gpus 1 (requests would shard across "
              "GPUs with no exchange; no multi-GPU run is made here)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe()
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

    ms = time_steps(step, args.steps, args.warmup)
    one_launch_ms = None
    if filt is not None:
        # Statistics kernel, per-row filter selection, sampler; the events sit
        # on the selection kernel, the call's longest (its algorithmic read is
        # one pass over every row, like the statistics kernel's).
        kernel_ms = time_streaming_kernel(step, args.steps, args.warmup)
    elif mode_of(case) == "stochastic":
        # The default schedule runs statistics and sampling in one launch; the
        # streaming roofline is taken on the statistics kernel of the
        # two-kernel schedule (same workload, same bytes), and the one-launch
        # kernel's own duration is reported beside it.
        one_launch_ms = time_streaming_kernel(step, args.steps, args.warmup)
        sv.spec_verify_set_schedule(_lib.SCHEDULE_TWO_KERNELS)
        try:
            kernel_ms = time_streaming_kernel(step, args.steps, args.warmup)
        finally:
            sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)
    else:
        kernel_ms = time_streaming_kernel(step, args.steps, args.warmup)
    k_avg = float(np.mean(kernel_ms))
    if mode_of(case) == "tree-stochastic":
        # the walk reads only the visited rows: the same outputs on every copy
        nbytes = tree_walk_bytes(case, step.nodes.cpu().numpy(), acc.cpu().numpy())
    rows = case.rows
    value = rows / (ms * 1e-3)
    achieved = nbytes / (k_avg * 1e-3) / 1e9
    n_acc = acc.cpu().numpy()
    src_hash = source_hash()
    traffic = load_traffic(args.workload, src_hash) if filt is None else None
    wname = case.name if filt is None else (
        f"{case.name}-topk{args.top_k}-topp{args.top_p:g}-minp{args.min_p:g}")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
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
            "seed": args.seed,
            **({"k": case.k} if mode_of(case) in ("stochastic", "greedy")
               else {"N": case.N, "P": case.P, "L": case.L}),
            **({"temperature": case.temperature}
               if mode_of(case) in ("stochastic", "tree-stochastic") else {}),
            **({} if filt is None else {"top_k": args.top_k, "top_p": args.top_p,
                                        "min_p": args.min_p}),
        },
        "hbm_gbps_whole_call": nbytes / (ms * 1e-3) / 1e9,
        "roofline": {
            "bound": "hbm",
            "kernel": ("filter selection kernel (filtered call)" if filt is not None else
                       "statistics kernel (two-kernel schedule)" if mode_of(case) == "stochastic"
                       else "tree walk kernel (each request's walk split over workgroups)"
                       if mode_of(case) == "tree-stochastic" else "argmax kernel"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel_us_mean": k_avg * 1e3,
            "kernel_us_p10_p90": [float(np.percentile(kernel_ms, 10)) * 1e3,
                                  float(np.percentile(kernel_ms, 90)) * 1e3],
            "algorithmic_bytes_per_launch": nbytes,
            "source_hash": src_hash,
        },
        "one_launch_kernel": None if one_launch_ms is None else {
            "us_mean": float(np.mean(one_launch_ms)) * 1e3,
            "algorithmic_gbps": nbytes / (float(np.mean(one_launch_ms)) * 1e-3) / 1e9,
            "note": "default schedule: statistics and sampling in one kernel",
        },
        "num_accepted_histogram": np.bincount(n_acc, minlength=(rows // case.B)).tolist(),
        "acceptance_length": float(n_acc.mean() + 1.0),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, filt)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
