"""GPU parity: stochastic verification with top-k / top-p / min-p applied alike to
every target and draft row (page "TensorRT-LLM source teardown (10)", "Rejection
sampling": both sides filtered identically), against the oracle's filtered
verification, through spec_verify_stochastic_filtered.

Same bar as the unfiltered calls (exact tokens on every request that is not
ambiguous, p/q within 1e-5), where a request is also ambiguous when one of its
filter decisions lies within 1e-9 of flipping (top-p: relative to the
survivors' mass; min-p: in logit units).  The GPU decides top-p with fast
weights (~1.5e-7 relative) only when its edge is more than 1e-6 away and
otherwise with fp64 weights (~1e-12), and computes min-p's threshold in fp64.

top_p and min_p cross the C ABI as float32, so the oracle is given exactly
those values."""
import numpy as np
import pytest
import torch

import draft_token_verification_verify_amd as sv
from draft_token_verification_verify_amd import _lib
from draft_token_verification_verify_amd import workloads as wl
from tests import gpu_helpers as H
from tests.oracle_pins import CHI2_DF7_P001, chi2_stat, lib_softmax, sample_from
import oracle

pytestmark = pytest.mark.gpu

FILTER_GUARD = 1e-9


def f32(x):
    return float(np.float32(x))


def run_filtered(case, top_k, top_p, min_p, *, workspace=None):
    dev = torch.device("cuda", 0)
    t = wl.to_device(case.target, case.dtype)
    d = wl.to_device(case.draft, case.dtype) if case.k > 0 else None
    x = wl.to_device(case.draft_tokens.astype(np.int32)) if case.k > 0 else None
    u = wl.to_device(case.uniforms.astype(np.float32))
    p = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    q = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    out, acc = sv.spec_verify_stochastic_filtered(t, d, x, u, case.temperature, top_k, top_p,
                                                  min_p, p_at_draft=p, q_at_draft=q,
                                                  workspace=workspace)
    torch.cuda.synchronize()
    return dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                p_at_draft=p.cpu().numpy(), q_at_draft=q.cpu().numpy())


def oracle_filtered(case, top_k, top_p, min_p):
    return oracle.stochastic(case.target, case.draft if case.k > 0 else None, case.draft_tokens,
                             case.uniforms, case.temperature, top_k=top_k, top_p=f32(top_p),
                             min_p=f32(min_p))


def check(case, top_k, top_p, min_p, label, max_ambiguous=None):
    gpu = run_filtered(case, top_k, top_p, min_p)
    ref = oracle_filtered(case, top_k, top_p, min_p)
    # min_p = 1 puts the threshold exactly on the row maximum (ln 1 = 0 on both
    # sides), which the oracle's min-p margin reports as 0; with no other
    # filter on, no decision of the filter is then in doubt.
    exact = min_p == 1.0 and top_p == 1.0 and not 0 < top_k < case.V
    amb, dis = H.compare_stochastic(gpu, ref, label=label,
                                    filter_band=None if exact else FILTER_GUARD)
    if max_ambiguous is None:
        max_ambiguous = max(1, 0.05 * case.B)
    assert amb <= max_ambiguous, f"{label}: {amb} ambiguous of {case.B}"
    # ambiguous requests that differ from the oracle: below 1e-4 of the rows,
    # as in every other stochastic suite (0 at these sizes)
    assert dis <= 1e-4 * case.rows, f"{label}: {dis} ambiguous requests differ"
    return gpu, ref


FILTERS = [
    ("topk1", 1, 1.0, 0.0),
    ("topk5", 5, 1.0, 0.0),
    ("topk50", 50, 1.0, 0.0),
    ("topp0.5", 0, 0.5, 0.0),
    ("topp0.9", 0, 0.9, 0.0),
    ("minp0.05", 0, 1.0, 0.05),
    ("minp1", 0, 1.0, 1.0),
    ("k50-p0.9", 50, 0.9, 0.0),
    ("k40-p0.8-minp0.02", 40, 0.8, 0.02),
    ("k3000-p0.7", 3000, 0.7, 0.0),
]

SHAPES = [
    ("f32-V1000-k3", lambda s: wl.gaussian_stochastic(s, 16, 3, 1000, "f32", target_sd=2.0,
                                                        draft_noise_sd=0.5)),
    ("bf16-V32000-k4", lambda s: wl.gaussian_stochastic(s, 8, 4, 32000, "bf16", target_sd=3.0,
                                                          draft_noise_sd=1.0)),
    ("f32-V50001-k2-unaligned", lambda s: wl.gaussian_stochastic(s, 5, 2, 50001, "f32",
                                                                   target_sd=2.0,
                                                                   draft_noise_sd=0.7)),
    ("c3-B6", lambda s: wl.c3(s, B=6)),
]


@pytest.mark.parametrize("fname,top_k,top_p,min_p", FILTERS, ids=[f[0] for f in FILTERS])
@pytest.mark.parametrize("sname,make", SHAPES, ids=[s[0] for s in SHAPES])
def test_filtered_parity(sname, make, fname, top_k, top_p, min_p):
    check(make(3), top_k, top_p, min_p, f"{sname}/{fname}")


def test_filtered_c4_rows():
    """fp32, a fresh Zipf permutation per row (C4's generator), a few requests."""
    case = wl.c4(5, B=4)
    check(case, 20, 0.9, 0.01, "c4-B4")


def test_k0_filters_the_bonus_row_only():
    case = wl.gaussian_stochastic(7, 32, 0, 4000, "bf16", target_sd=2.0, draft_noise_sd=1.0)
    check(case, 10, 0.9, 0.0, "k0")


def test_filters_off_is_the_plain_call():
    case = wl.gaussian_stochastic(11, 16, 3, 5000, "bf16", target_sd=2.0, draft_noise_sd=1.0)
    plain = H.run_stochastic(case)
    for top_k in (0, case.V, case.V + 5):
        off = run_filtered(case, top_k, 1.0, 0.0)
        for key in plain:
            np.testing.assert_array_equal(off[key], plain[key], err_msg=f"{key}, top_k={top_k}")


def _flat_case(seed, B, k, V, dtype, width):
    """Logits in [0, width): a whole row falls into the top weight bin, so the
    selection has to narrow it by key digits before it fits in LDS."""
    rng = np.random.default_rng(seed)
    t32 = rng.random((B, k + 1, V), dtype=np.float32) * np.float32(width)
    d32 = (t32[:, :k] + rng.random((B, k, V), dtype=np.float32) * np.float32(width)).astype(
        np.float32)
    return wl.StochasticCase(f"flat-{dtype}", B, k, V, dtype, 1.0, wl._finish(t32, dtype),
                             wl._finish(d32, dtype), rng.integers(0, V, (B, k)).astype(np.int32),
                             rng.random((B, k + 1), dtype=np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("top_k,top_p", [(100, 1.0), (20000, 1.0), (0, 0.5), (30000, 0.3)])
def test_boundary_bin_larger_than_lds(dtype, top_k, top_p):
    case = _flat_case(21, 6, 2, 32768, dtype, 0.01)
    check(case, top_k, top_p, 0.0, f"flat-{dtype}-k{top_k}-p{top_p}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("top_k,top_p", [(5000, 1.0), (0, 0.4), (0, 0.8), (15000, 0.5)])
def test_large_tie_group_at_the_boundary(dtype, top_k, top_p):
    """20000 tokens share the row maximum (more than fit in LDS): the thresholds
    land inside the tie group and every tied token is kept."""
    rng = np.random.default_rng(31)
    B, k, V = 2, 2, 32768
    t32 = (rng.random((B, k + 1, V), dtype=np.float32) - np.float32(2.0)).astype(np.float32)
    d32 = (rng.random((B, k, V), dtype=np.float32) - np.float32(2.0)).astype(np.float32)
    for a in (t32, d32):
        idx = rng.permuted(np.broadcast_to(np.arange(V), a.shape[:-1] + (V,)), axis=-1)[..., :20000]
        np.put_along_axis(a, idx, np.float32(1.0), axis=-1)
    case = wl.StochasticCase("ties", B, k, V, dtype, 1.0, wl._finish(t32, dtype),
                             wl._finish(d32, dtype), rng.integers(0, V, (B, k)).astype(np.int32),
                             rng.random((B, k + 1), dtype=np.float32))
    check(case, top_k, top_p, 0.0, f"ties-{dtype}-k{top_k}-p{top_p}")


def test_masked_tokens_and_top_k_beyond_the_finite_ones():
    """-inf logits (masked vocabulary) stay at probability 0; top_k larger than
    the number of finite logits keeps all of them."""
    case = wl.gaussian_stochastic(41, 6, 3, 4096, "f32", target_sd=2.0, draft_noise_sd=0.5)
    rng = np.random.default_rng(41)
    for a in (case.target, case.draft):
        a[..., 3000:] = -np.inf
        a[..., rng.integers(0, 3000, 200)] = -np.inf
    keep = np.isfinite(case.draft[np.arange(case.B)[:, None], np.arange(case.k)[None, :],
                                  case.draft_tokens])
    case.draft_tokens = np.where(keep, case.draft_tokens, 0).astype(np.int32)
    for top_k, top_p, min_p in ((3500, 1.0, 0.0), (3500, 0.9, 0.0), (10, 0.5, 0.1)):
        check(case, top_k, top_p, min_p, f"masked-k{top_k}")


@pytest.mark.parametrize("mode", [_lib.MODE_STOCHASTIC, _lib.MODE_STOCHASTIC_FILTERED])
def test_workspace_is_zero_after_filtered_calls(mode):
    case = wl.gaussian_stochastic(5, 8, 3, 6000, "bf16", target_sd=2.0, draft_noise_sd=1.0)
    dev = torch.device("cuda", 0)
    ws = torch.zeros(sv.spec_verify_workspace_bytes(mode, case.B, case.k + 1, case.V, _lib.BF16),
                     dtype=torch.uint8, device=dev)
    for top_k, top_p, min_p in ((5, 1.0, 0.0), (0, 0.9, 0.05), (30, 0.7, 0.0), (0, 1.0, 0.1)):
        run_filtered(case, top_k, top_p, min_p, workspace=ws)
        assert int(torch.count_nonzero(ws)) == 0


def _workspace(case, mode):
    dt = _lib.BF16 if case.dtype == "bf16" else _lib.F32
    return torch.zeros(sv.spec_verify_workspace_bytes(mode, case.B, case.k + 1, case.V, dt),
                       dtype=torch.uint8, device=torch.device("cuda", 0))


@pytest.mark.parametrize("sname,make", SHAPES, ids=[s[0] for s in SHAPES])
def test_candidates_and_row_passes_give_the_same_bits(sname, make):
    """A workspace with room for the statistics' candidates and one without
    (the filter then reads every row itself) give identical outputs: the
    thresholds and kept masses come from order-free fixed-point sums."""
    case = make(4)
    small, large = _workspace(case, _lib.MODE_STOCHASTIC), _workspace(
        case, _lib.MODE_STOCHASTIC_FILTERED)
    for _, top_k, top_p, min_p in FILTERS:
        a = run_filtered(case, top_k, top_p, min_p, workspace=small)
        b = run_filtered(case, top_k, top_p, min_p, workspace=large)
        for key in a:
            np.testing.assert_array_equal(a[key], b[key], err_msg=f"{key} {top_k} {top_p} {min_p}")


def test_row_passes_parity():
    """The filter that reads every row (workspace without candidate room)
    against the oracle."""
    case = wl.c3(6, B=6)
    ws = _workspace(case, _lib.MODE_STOCHASTIC)
    for _, top_k, top_p, min_p in FILTERS:
        gpu = run_filtered(case, top_k, top_p, min_p, workspace=ws)
        ref = oracle_filtered(case, top_k, top_p, min_p)
        exact = min_p == 1.0 and top_p == 1.0 and not 0 < top_k < case.V
        H.compare_stochastic(gpu, ref, label=f"rows/{top_k}/{top_p}/{min_p}",
                             filter_band=None if exact else FILTER_GUARD)


def test_repeat_calls_are_bit_identical():
    case = wl.c3(2, B=4)
    a = run_filtered(case, 50, 0.9, 0.0)
    b = run_filtered(case, 50, 0.9, 0.0)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_filtered_output_distributed_as_filtered_p():
    """Chi-squared, V = 8, top-k 5 and top-p 0.9 on both sides, drafts drawn from
    the filtered q: the first emitted token is distributed as the filtered p
    (filtered distributions computed here from a sort of the library softmax)."""
    rng = np.random.default_rng(53)
    V, trials = 8, 400_000
    tl = rng.normal(0, 1.2, (2, V)).astype(np.float32)
    dl = (tl[:1] + rng.normal(0, 1.0, (1, V))).astype(np.float32)

    def filtered(logits):
        p = lib_softmax(logits)
        order = np.argsort(-logits, kind="stable")
        keep = np.zeros(V, bool)
        keep[order[:5]] = True
        p5 = np.where(keep, p, 0.0) / p[keep].sum()
        cum = np.cumsum(p5[order])
        cut = order[: int(np.searchsorted(cum, f32(0.9))) + 1]
        out = np.zeros(V)
        out[cut] = p[cut]
        return out / out.sum()

    pf, qf = filtered(tl[0]), filtered(dl[0])
    x = sample_from(rng, qf, trials).reshape(trials, 1).astype(np.int32)
    u = rng.random((trials, 2), dtype=np.float32)
    t = np.broadcast_to(tl, (trials, 2, V)).copy()
    d = np.broadcast_to(dl, (trials, 1, V)).copy()
    case = wl.StochasticCase("chi2", trials, 1, V, "f32", 1.0, t, d, x, u)
    gpu = run_filtered(case, 5, 0.9, 0.0)
    assert chi2_stat(np.bincount(gpu["out_tokens"][:, 0], minlength=V), pf) < CHI2_DF7_P001


def _top_p_at_group_edge(case, b, row, near=0.9):
    """A float32 top_p whose target mass for target row `row` of request b lies
    1e-9 .. 1e-7 (relative to the row's mass) from a group edge: the fp64
    cumulative masses of the row's descending groups of equal logits, the
    group end nearest `near`, and the nearest float32 to it at least 2e-9
    away."""
    r = case.target[b, row]
    x = (wl.bits_to_float(r) if case.dtype == "bf16" else r).astype(np.float64)
    w = np.exp2((x - x.max()) * (np.log2(np.e) / float(np.float32(case.temperature))))
    vals, inv = np.unique(-x, return_inverse=True)  # ascending -x: descending logits
    cum = np.cumsum(np.bincount(inv, weights=w)) / w.sum()
    f = float(cum[np.argmin(np.abs(cum - near))])
    p = np.float32(f)
    if abs(float(p) - f) < 2e-9:
        p = np.nextafter(p, np.float32(1.0 if float(p) >= f else 0.0))
    return float(p)


@pytest.mark.parametrize("mode", [_lib.MODE_STOCHASTIC, _lib.MODE_STOCHASTIC_FILTERED])
def test_top_p_decided_near_a_group_edge(mode):
    """Top-p alone with the target 1e-9 .. 1e-7 from a group edge on one row:
    closer than the statistics' row mass can tell (~1e-5), so the decision
    comes from the candidate gather's fp64 tail masses (large workspace) or the
    selection's own fp64 tail pass (small workspace); both must agree with the
    oracle on that request."""
    case = wl.c3(8, B=4)
    top_p = _top_p_at_group_edge(case, 1, 0)
    ref = oracle_filtered(case, 0, top_p, 0.0)
    assert 1e-9 <= ref["filter_margins"][1] < 1e-6  # the hard case is really there
    gpu = run_filtered(case, 0, top_p, 0.0, workspace=_workspace(case, mode))
    H.compare_stochastic(gpu, ref, label=f"edge-{mode}", filter_band=FILTER_GUARD)
    assert gpu["num_accepted"][1] == ref["num_accepted"][1]
    np.testing.assert_array_equal(gpu["out_tokens"][1], ref["out_tokens"][1])
