"""Every verification call captured in a HIP graph: each replay gives the eager
call's bits (the calls record no memset node; their exchange areas are cleared
by their own kernels, so a replay finds them as the eager call left them).
Replays alternate with eager calls and synchronisations, and every replay is
checked."""
import numpy as np
import pytest
import torch

import draft_token_verification_verify_amd as sv
from draft_token_verification_verify_amd import workloads as wl
from draft_token_verification_verify_amd.workloads import to_device as to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _check_replays(call, outputs, label):
    """call() issues one verification on the current stream into `outputs`."""
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # the capture stream's workspace exists before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in outputs:
            o.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(o, r), f"{label}: replay {rep}, output {i} differs from eager"
        call()  # eager work between replays
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(o, r), f"{label}: eager call after replay {rep}, output {i}"


STOCHASTIC = [
    ("c1", lambda: wl.c1(3)),
    ("c2", lambda: wl.c2_stochastic(4)),
    ("B32 k3 V65536 bf16 (one launch)",
     lambda: wl.gaussian_stochastic(5, 32, 3, 65536, "bf16", target_sd=3.0, draft_noise_sd=1.0)),
]


@pytest.mark.parametrize("make", [m for _, m in STOCHASTIC], ids=[n for n, _ in STOCHASTIC])
def test_stochastic_call_replays(make):
    case = make()
    dev = torch.device("cuda", 0)
    t = to_dev(case.target, case.dtype)
    d = to_dev(case.draft, case.dtype)
    x = to_dev(case.draft_tokens.astype(np.int32))
    u = to_dev(case.uniforms.astype(np.float32))
    out = torch.empty((case.B, case.k + 1), dtype=torch.int32, device=dev)
    acc = torch.empty((case.B,), dtype=torch.int32, device=dev)
    p = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    q = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)

    def call():
        sv.spec_verify_stochastic(t, d, x, u, case.temperature, out_tokens=out, num_accepted=acc,
                                  p_at_draft=p, q_at_draft=q)

    _check_replays(call, [out, acc, p, q], case.name)


def test_filtered_call_replays():
    case = wl.gaussian_stochastic(6, 8, 3, 32000, "bf16", target_sd=3.0, draft_noise_sd=1.0)
    dev = torch.device("cuda", 0)
    t = to_dev(case.target, case.dtype)
    d = to_dev(case.draft, case.dtype)
    x = to_dev(case.draft_tokens.astype(np.int32))
    u = to_dev(case.uniforms.astype(np.float32))
    out = torch.empty((case.B, case.k + 1), dtype=torch.int32, device=dev)
    acc = torch.empty((case.B,), dtype=torch.int32, device=dev)

    def call():
        sv.spec_verify_stochastic_filtered(t, d, x, u, case.temperature, 20, 0.9, 0.01,
                                           out_tokens=out, num_accepted=acc)

    _check_replays(call, [out, acc], "filtered top-k 20 top-p 0.9 min-p 0.01")


def test_greedy_call_replays():
    case = wl.c2_greedy(7)
    dev = torch.device("cuda", 0)
    t = to_dev(case.target, case.dtype)
    x = to_dev(case.draft_tokens.astype(np.int32))
    out = torch.empty((case.B, case.k + 1), dtype=torch.int32, device=dev)
    acc = torch.empty((case.B,), dtype=torch.int32, device=dev)

    def call():
        sv.spec_verify_greedy(t, x, out_tokens=out, num_accepted=acc)

    _check_replays(call, [out, acc], case.name)


def test_tree_call_replays():
    case = wl.random_tree_case(8, 4, 20, 4, 32000, "bf16")
    dev = torch.device("cuda", 0)
    t = to_dev(case.target, case.dtype)
    nt = to_dev(case.node_tokens.astype(np.int32))
    pa = to_dev(case.paths.astype(np.int32))
    out = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)
    acc = torch.empty((case.B,), dtype=torch.int32, device=dev)
    best = torch.empty((case.B,), dtype=torch.int32, device=dev)
    nodes = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)

    def call():
        sv.spec_verify_tree(t, nt, pa, out_tokens=out, num_accepted=acc, best_path=best,
                            accepted_nodes=nodes)

    _check_replays(call, [out, acc, best, nodes], case.name)


def test_tree_stochastic_call_replays():
    case = wl.stochastic_tree_case(9, 4, 20, 4, 32000, "bf16")
    dev = torch.device("cuda", 0)
    t = to_dev(case.target, case.dtype)
    d = to_dev(case.draft, case.dtype)
    nt = to_dev(case.node_tokens.astype(np.int32))
    pa = to_dev(case.paths.astype(np.int32))
    u = to_dev(case.uniforms.astype(np.float32))
    out = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)
    acc = torch.empty((case.B,), dtype=torch.int32, device=dev)
    nodes = torch.empty((case.B, case.L), dtype=torch.int32, device=dev)

    def call():
        # the give-up check reads num_accepted on the host: not in a capture
        sv.spec_verify_tree_stochastic(t, d, nt, pa, u, case.temperature, out_tokens=out,
                                       num_accepted=acc, accepted_nodes=nodes, check=False)

    _check_replays(call, [out, acc, nodes], case.name)
