"""GPU parity: stochastic tree verification (each accepted node's children tested
in ascending order against the residual left by their rejected siblings; page
"05 - TensorRT-LLM speculative decoding and auto-deploy", "Target-model
verification: tree attention and batched parallelism") and the accepted-row
gather (page "TensorRT-LLM source teardown (10)", KV rewind, fourth step),
against the oracle, through spec_verify_tree_stochastic and
spec_verify_gather_rows.

Bar: out_tokens, num_accepted and accepted_nodes equal the oracle's on every
request none of whose decisions (tests taken, final draw) lies within 1e-6 of
its boundary; ambiguous requests that differ stay below 1e-4 of the rows."""
import numpy as np
import pytest
import torch

import draft_token_verification_verify_amd as sv
from draft_token_verification_verify_amd import workloads as wl
from tests import gpu_helpers as H
from tests.oracle_pins import CHI2_DF7_P001, chi2_stat, lib_softmax, sample_from
import oracle

pytestmark = pytest.mark.gpu


def run_tree_stochastic(case, split=True, workspace=None, check=True):
    t = wl.to_device(case.target, case.dtype)
    d = wl.to_device(case.draft, case.dtype)
    nt = wl.to_device(case.node_tokens.astype(np.int32))
    pa = wl.to_device(case.paths.astype(np.int32))
    u = wl.to_device(case.uniforms.astype(np.float32))
    out, acc, nodes = sv.spec_verify_tree_stochastic(t, d, nt, pa, u, case.temperature,
                                                     split=split, workspace=workspace,
                                                     check=check)
    torch.cuda.synchronize()
    return dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                accepted_nodes=nodes.cpu().numpy())


def oracle_tree_stochastic(case):
    return oracle.tree_stochastic(case.target, case.draft, case.node_tokens, case.paths,
                                  case.uniforms, case.temperature)


def compare(gpu, ref, label, rows):
    amb = oracle.ambiguous_requests(ref["margins"], H.GUARD)
    same = ((gpu["num_accepted"] == ref["num_accepted"])
            & np.all(gpu["out_tokens"] == ref["out_tokens"], axis=1)
            & np.all(gpu["accepted_nodes"] == ref["accepted_nodes"], axis=1))
    bad = np.nonzero(~same & ~amb)[0]
    assert bad.size == 0, (
        f"{label}: {bad.size} non-ambiguous requests differ, first {bad[:5]}: gpu "
        f"{gpu['out_tokens'][bad[:3]]} / {gpu['accepted_nodes'][bad[:3]]} vs oracle "
        f"{ref['out_tokens'][bad[:3]]} / {ref['accepted_nodes'][bad[:3]]}")
    assert int((amb & ~same).sum()) <= max(1e-4 * rows, 0), f"{label}: ambiguous requests differ"
    return int(amb.sum())


CASES = [
    ("f32-V1000-N12-d4", lambda s: wl.stochastic_tree_case(s, 24, 12, 4, 1000, "f32",
                                                           target_sd=2.0, draft_noise_sd=0.7)),
    ("bf16-V32000-N30-d5", lambda s: wl.stochastic_tree_case(s, 8, 30, 5, 32000, "bf16",
                                                             target_sd=3.0, draft_noise_sd=1.0)),
    ("f32-V5001-N20-d3-unaligned", lambda s: wl.stochastic_tree_case(
        s, 8, 20, 3, 5001, "f32", target_sd=2.0, draft_noise_sd=0.5, temperature=0.7)),
    ("c5-shape-B6", lambda s: wl.stochastic_tree_case(s, 6, 60, 6, 128256, "bf16",
                                                      target_sd=3.0, draft_noise_sd=1.0)),
    ("f32-V9-N40-d6", lambda s: wl.stochastic_tree_case(s, 64, 40, 6, 9, "f32", target_sd=1.0,
                                                        draft_noise_sd=1.0, max_children=4)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("seed", [0, 1])
def test_tree_stochastic_parity(name, make, seed):
    case = make(seed)
    gpu = run_tree_stochastic(case)
    ref = oracle_tree_stochastic(case)
    compare(gpu, ref, name, case.rows)
    for b in range(case.B):  # accepted nodes form a chain from the root
        s = int(gpu["num_accepted"][b])
        prev = 0
        for j in range(s):
            n = int(gpu["accepted_nodes"][b, j])
            assert case.parents[b, n] == prev
            prev = n


def _chain_case(seed, B, k, V, dtype):
    """A single-chain tree over the rows of a linear stochastic case."""
    lin = wl.gaussian_stochastic(seed, B, k, V, dtype, target_sd=2.0, draft_noise_sd=1.0)
    draft = np.concatenate([lin.draft, lin.draft[:, :1]], axis=1)  # row k: a leaf, not read
    tok = np.concatenate([np.zeros((B, 1), np.int32), lin.draft_tokens], axis=1)
    paths = np.full((B, 2, k + 1), -1, np.int32)
    paths[:, 0] = np.arange(k + 1)
    parents = np.arange(-1, k, dtype=np.int32)[None].repeat(B, 0)
    tree = wl.StochasticTreeCase("chain", B, k, 2, k + 1, V, dtype, lin.temperature, lin.target,
                                 draft, tok, paths, lin.uniforms, parents)
    return lin, tree


@pytest.mark.parametrize("dtype,V,k", [("bf16", 32000, 4), ("f32", 777, 6)])
def test_chain_tree_matches_the_linear_call(dtype, V, k):
    lin, tree = _chain_case(5, 32, k, V, dtype)
    g_tree = run_tree_stochastic(tree)
    ref = H.oracle_stochastic(lin)
    amb = oracle.ambiguous_requests(ref["margins"], H.GUARD)
    same = ((g_tree["num_accepted"] == ref["num_accepted"])
            & np.all(g_tree["out_tokens"] == ref["out_tokens"], axis=1))
    assert np.all(same | amb)


def test_root_alone_and_out_of_range_ids():
    case = wl.stochastic_tree_case(9, 16, 10, 3, 600, "f32", target_sd=2.0, draft_noise_sd=1.0)
    case.paths[:4] = -1  # no usable row: the final token comes from the root's row
    case.node_tokens[4:8, 1:] = case.V + 3  # every child out of range: all rejected
    gpu = run_tree_stochastic(case)
    ref = oracle_tree_stochastic(case)
    compare(gpu, ref, "root-alone", case.rows)
    assert np.all(gpu["num_accepted"][:8] == 0)


def test_identical_draft_walks_first_children():
    case = wl.stochastic_tree_case(13, 16, 20, 4, 3000, "bf16", target_sd=2.0, draft_noise_sd=0.0)
    case.draft = case.target.copy()
    gpu = run_tree_stochastic(case)
    ref = oracle_tree_stochastic(case)
    compare(gpu, ref, "identical", case.rows)
    assert np.all(gpu["num_accepted"] == case.L - 1)


def test_repeat_calls_are_bit_identical():
    case = wl.stochastic_tree_case(3, 8, 30, 5, 20000, "bf16")
    a = run_tree_stochastic(case)
    b = run_tree_stochastic(case)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_first_token_distributed_as_p():
    """Chi-squared on the GPU: three children drawn independently from q at the
    root, V = 8, 300 000 requests; the first emitted token is distributed as p."""
    rng = np.random.default_rng(67)
    V, m, trials = 8, 3, 300_000
    tl = rng.normal(0, 1.2, (m + 1, V)).astype(np.float32)
    dl = (tl + rng.normal(0, 1.0, (m + 1, V))).astype(np.float32)
    p = lib_softmax(tl[0])
    q = lib_softmax(dl[0])
    tok = np.zeros((trials, m + 1), np.int32)
    tok[:, 1:] = sample_from(rng, q, trials * m).reshape(trials, m)
    paths = np.full((trials, m, 2), -1, np.int32)
    for c in range(1, m + 1):
        paths[:, c - 1] = [0, c]
    u = rng.random((trials, m + 1), dtype=np.float32)
    t = np.broadcast_to(tl, (trials, m + 1, V)).copy()
    d = np.broadcast_to(dl, (trials, m + 1, V)).copy()
    parents = np.array([-1] + [0] * m, np.int32)[None].repeat(trials, 0)
    case = wl.StochasticTreeCase("chi2", trials, m, m, 2, V, "f32", 1.0, t, d, tok, paths, u,
                                 parents)
    gpu = run_tree_stochastic(case)
    assert chi2_stat(np.bincount(gpu["out_tokens"][:, 0], minlength=V), p) < CHI2_DF7_P001


@pytest.mark.parametrize("row_shape,dtype", [((2, 8, 64), torch.bfloat16), ((3,), torch.int16),
                                             ((5, 7), torch.float32)])
def test_gather_rows(row_shape, dtype):
    case = wl.stochastic_tree_case(21, 8, 30, 5, 4000, "bf16")
    gpu = run_tree_stochastic(case)
    B, N1, L = case.B, case.N + 1, case.L
    gen = torch.Generator().manual_seed(5)
    src = torch.randn((B, N1) + row_shape, generator=gen).to(dtype)
    dst0 = torch.full((B, L) + row_shape, -3).to(dtype)
    want = oracle.gather_rows(src.view(B, N1, -1).float().numpy(), gpu["accepted_nodes"],
                              gpu["num_accepted"], dst0.view(B, L, -1).float().numpy())
    dev = torch.device("cuda", 0)
    nodes = torch.from_numpy(gpu["accepted_nodes"]).to(dev)
    acc = torch.from_numpy(gpu["num_accepted"]).to(dev)
    dst = dst0.to(dev)
    sv.spec_verify_gather_rows(src.to(dev), nodes, acc, dst)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dst.cpu().view(B, L, -1).float().numpy(), want)


@pytest.mark.parametrize("name,make", [CASES[1], CASES[3]], ids=[CASES[1][0], CASES[3][0]])
def test_tree_stochastic_parity_one_workgroup(name, make):
    """Without a workspace every request's walk runs in one workgroup (with
    one, the C5-shaped case is split over 8)."""
    from draft_token_verification_verify_amd import _lib
    assert sv.spec_verify_tree_stochastic_split(6, 128256, _lib.BF16) == 8
    case = make(0)
    gpu = run_tree_stochastic(case, split=False)
    compare(gpu, oracle_tree_stochastic(case), name + "-1wg", case.rows)


def test_benchmarked_workload_full_size():
    """The stochastic-tree workload the benchmark times, at its full size and in
    its launch configuration: B=32 trees of 60 nodes, depth 6, V=128256 bf16,
    each request's walk split over 8 workgroups; every request against the
    oracle."""
    from draft_token_verification_verify_amd import _lib
    case = wl.stochastic_tree_case(0, 32, 60, 6, 128256, "bf16", target_sd=3.0,
                                   draft_noise_sd=1.0)
    assert sv.spec_verify_tree_stochastic_split(case.B, case.V, _lib.BF16) == 8
    gpu = run_tree_stochastic(case)
    assert np.all(gpu["num_accepted"] >= 0)
    amb = compare(gpu, oracle_tree_stochastic(case), "c5-shape-B32", case.rows)
    print(f"c5-shape-B32: {amb} ambiguous requests")


def test_split_walk_leaves_the_workspace_zero():
    """Split walks of two shapes in a row through one workspace: the exchange
    areas are cleared by each call's last workgroup (and no request gave up
    waiting: num_accepted >= 0)."""
    from draft_token_verification_verify_amd import _lib
    dev = torch.device("cuda", 0)
    ws = torch.zeros(sv.spec_verify_workspace_bytes(_lib.MODE_TREE_STOCHASTIC, 16, 61, 32000,
                                                    _lib.BF16), dtype=torch.uint8, device=dev)
    for case in (wl.stochastic_tree_case(4, 16, 60, 6, 32000, "bf16"),
                 wl.stochastic_tree_case(5, 8, 30, 5, 20000, "bf16")):
        tiles = -(-case.V // 8192)  # the walk reads rows in tiles of 8192 logits
        assert sv.spec_verify_tree_stochastic_split(case.B, case.V, _lib.BF16) == tiles  # 4, then 3
        gpu = run_tree_stochastic(case, workspace=ws)
        assert np.all(gpu["num_accepted"] >= 0)
        compare(gpu, oracle_tree_stochastic(case), "ws", case.rows)
        assert int(torch.count_nonzero(ws)) == 0


def test_split_walk_gives_up_cleanly_when_forced():
    """The split walk's failure path, forced from the host: with the poll limit
    of an exchange word at 0, the workgroups of a request give up waiting for
    each other.  The kernel still ends; every request is either marked
    num_accepted = -2 (at least one is) or, having given up on no exchange,
    matches the oracle; and the workspace is zero afterwards.  With the default
    limit back, the same workspace gives full parity again."""
    from draft_token_verification_verify_amd import _lib
    lib = _lib.load()
    case = wl.stochastic_tree_case(3, 6, 60, 6, 128256, "bf16", target_sd=3.0, draft_noise_sd=1.0)
    assert sv.spec_verify_tree_stochastic_split(case.B, case.V, _lib.BF16) == 8
    n1 = case.node_tokens.shape[1]
    ws = torch.zeros(sv.spec_verify_workspace_bytes(_lib.MODE_TREE_STOCHASTIC, case.B, n1, case.V,
                                                    _lib.BF16), dtype=torch.uint8, device="cuda")
    ref = oracle_tree_stochastic(case)
    prev = lib.spec_verify_debug_tree_spin_limit(0)
    try:
        gpu = run_tree_stochastic(case, workspace=ws, check=False)
    finally:
        assert lib.spec_verify_debug_tree_spin_limit(-1) == 0
    assert prev == 1 << 20
    acc = gpu["num_accepted"]
    # the binding's check reports the given-up requests
    with pytest.raises(sv.SpecVerifyError, match="gave up"):
        sv.check_tree_stochastic_result(torch.from_numpy(acc))
    assert np.all((acc == -2) | (acc >= 0)), acc
    assert np.any(acc == -2), acc
    amb = oracle.ambiguous_requests(ref["margins"], H.GUARD)
    for b in np.nonzero((acc >= 0) & ~amb)[0]:
        assert acc[b] == ref["num_accepted"][b], b
        assert np.array_equal(gpu["out_tokens"][b], ref["out_tokens"][b]), b
    assert int(torch.count_nonzero(ws)) == 0
    gpu = run_tree_stochastic(case, workspace=ws)
    assert np.all(gpu["num_accepted"] >= 0)
    compare(gpu, ref, "after", case.rows)
    assert int(torch.count_nonzero(ws)) == 0


def test_split_walks_on_two_streams_at_once():
    """Two split walks launched at once on two streams, each with its own
    workspace and each large enough to fill the device on its own.  A walk's
    groups are formed by arrival, so neither waits for workgroups that the
    other keeps from starting: both end without giving up and match the
    oracle, and both workspaces are zero afterwards."""
    from draft_token_verification_verify_amd import _lib
    V = 65536  # 8 tiles per row
    full = [b for b in range(1, 129) if sv.spec_verify_tree_stochastic_split(b, V, _lib.BF16) == 8]
    if not full or max(full) > 64:
        pytest.skip("device capacity outside the range this test sizes for")
    B = max(full)  # B * 8 workgroups: the most the device holds at once
    cases = [wl.stochastic_tree_case(s, B, 30, 5, V, "bf16", target_sd=3.0, draft_noise_sd=1.0)
             for s in (21, 22)]
    dev = torch.device("cuda", 0)
    streams = [torch.cuda.Stream(device=dev) for _ in cases]
    inputs, outs, spaces = [], [], []
    for case in cases:
        inputs.append((wl.to_device(case.target, case.dtype), wl.to_device(case.draft, case.dtype),
                       wl.to_device(case.node_tokens.astype(np.int32)),
                       wl.to_device(case.paths.astype(np.int32)),
                       wl.to_device(case.uniforms.astype(np.float32))))
        spaces.append(torch.zeros(sv.spec_verify_workspace_bytes(
            _lib.MODE_TREE_STOCHASTIC, B, case.node_tokens.shape[1], V, _lib.BF16),
            dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    for case, (t, d, nt, pa, u), ws, st in zip(cases, inputs, spaces, streams):
        with torch.cuda.stream(st):
            outs.append(sv.spec_verify_tree_stochastic(t, d, nt, pa, u, case.temperature,
                                                       workspace=ws))
    torch.cuda.synchronize()
    for case, (out, acc, nodes), ws in zip(cases, outs, spaces):
        gpu = dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                   accepted_nodes=nodes.cpu().numpy())
        assert np.all(gpu["num_accepted"] >= 0)
        compare(gpu, oracle_tree_stochastic(case), "two-streams", case.rows)
        assert int(torch.count_nonzero(ws)) == 0


def test_split_walk_with_several_tiles_per_workgroup():
    """Enough requests over a 128256-token vocabulary (16 tiles per row) that
    fewer workgroups per request fit on the device than there are tiles, so
    each takes several (k = g, g + G, ...)."""
    from draft_token_verification_verify_amd import _lib
    V = 128256
    B = next((b for b in (64, 96, 128, 192, 256)
              if 2 <= sv.spec_verify_tree_stochastic_split(b, V, _lib.BF16) < 8), None)
    if B is None:
        pytest.skip("no batch size gives 2..7 workgroups per request on this device")
    case = wl.stochastic_tree_case(17, B, 6, 3, V, "bf16", target_sd=3.0, draft_noise_sd=1.0)
    gpu = run_tree_stochastic(case)
    assert np.all(gpu["num_accepted"] >= 0)
    compare(gpu, oracle_tree_stochastic(case), "64req", case.rows)
