"""GPU parity: stochastic verification through the C ABI against the fp64 oracle.

Bar: out_tokens and num_accepted equal to the oracle on every request none of
whose decisions lies within 1e-6 of its threshold or CDF boundary; requests that
do (ambiguous) may differ, and the ones that differ are counted and must stay
below 1e-4 of the rows; p(x_i) and q(x_i) within 1e-5 relative.  The ambiguous
count itself is reported, not bounded: with V ~ 10^5 CDF edges a 1e-6 band
around each edge covers a few percent of [0, 1) on heavy-tailed rows.
"""
import functools

import numpy as np
import pytest
import torch

import draft_token_verification_verify_amd as sv
from draft_token_verification_verify_amd import workloads as wl
from tests import gpu_helpers as H
from tests.oracle_pins import CHI2_DF7_P001, chi2_stat, lib_softmax, sample_from

pytestmark = pytest.mark.gpu


# Cases too large to run a third time: the interleaved one-launch layout is
# what the default schedule already uses for the 1.7 GB workload.
_NOT_INTERLEAVED = {"test_c4_full_size", "test_c3_disagreements_over_many_seeds"}


@pytest.fixture(autouse=True, params=["auto", "two-kernels", "interleaved"])
def schedule(request):
    """Every case runs under the default one-launch schedule (two kernels where
    rows are not 16-byte aligned), under the two-kernel schedule, and under the
    one-launch schedule with each request's sampling workgroups right behind its
    statistics workgroups (they poll statistics still being computed)."""
    from draft_token_verification_verify_amd import _lib

    if request.param == "interleaved" and request.node.originalname in _NOT_INTERLEAVED:
        pytest.skip("covered by the default schedule's interleaved layout at this size")
    sv.spec_verify_set_schedule({"auto": _lib.SCHEDULE_AUTO,
                                 "two-kernels": _lib.SCHEDULE_TWO_KERNELS,
                                 "interleaved": _lib.SCHEDULE_INTERLEAVED}[request.param])
    yield request.param
    sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)


def check(case, rows=None):
    gpu = H.run_stochastic(case)
    ref = H.oracle_stochastic(case, rows)
    amb, dis = H.compare_stochastic(gpu, ref, rows, case.name)
    n_rows = case.B * (case.k + 1) if rows is None else len(rows) * (case.k + 1)
    print(f"{case.name}: {amb} ambiguous requests, {dis} differ (rows {n_rows})")
    assert dis <= 1e-4 * n_rows, f"{case.name}: {dis} ambiguous requests differ"
    return gpu, ref, amb, dis


SMALL = [
    # (name, factory) -- sizes that span several chunks and end in a ragged chunk
    ("bf16-V40000-k3", lambda s: wl.gaussian_stochastic(s, 4, 3, 40000, "bf16", target_sd=3.0,
                                                        draft_noise_sd=1.0)),
    ("f32-V50001-k2-unaligned", lambda s: wl.gaussian_stochastic(s, 3, 2, 50001, "f32",
                                                                 target_sd=2.0,
                                                                 draft_noise_sd=0.7)),
    ("bf16-V77777-k4-unaligned", lambda s: wl.gaussian_stochastic(s, 2, 4, 77777, "bf16",
                                                                  target_sd=2.0,
                                                                  draft_noise_sd=1.0,
                                                                  temperature=1.7)),
    ("f32-V33000-k0", lambda s: wl.gaussian_stochastic(s, 5, 0, 33000, "f32", target_sd=2.0,
                                                       draft_noise_sd=1.0)),
    ("bf16-V6000-k8", lambda s: wl.gaussian_stochastic(s, 6, 8, 6000, "bf16", target_sd=1.5,
                                                       draft_noise_sd=0.3, temperature=0.6)),
    ("zipf-bf16-V128256-B8", lambda s: wl.c3(s, B=8)),
    ("zipf-f32-V151936-B4", lambda s: wl.c4(s, B=4)),
    ("f32-V1-k3", lambda s: wl.gaussian_stochastic(s, 3, 3, 1, "f32", target_sd=1.0,
                                                   draft_noise_sd=1.0)),
    ("f32-V9-k5", lambda s: wl.gaussian_stochastic(s, 64, 5, 9, "f32", target_sd=1.0,
                                                   draft_noise_sd=1.0)),
    ("bf16-V20000-k3-T0.001", lambda s: wl.gaussian_stochastic(s, 8, 3, 20000, "bf16",
                                                               target_sd=2.0,
                                                               draft_noise_sd=0.5,
                                                               temperature=1e-3)),
    ("f32-V20000-k3-T37.5", lambda s: wl.gaussian_stochastic(s, 8, 3, 20000, "f32",
                                                             target_sd=2.0,
                                                             draft_noise_sd=0.5,
                                                             temperature=37.5)),
]


@pytest.mark.parametrize("name,factory", SMALL, ids=[n for n, _ in SMALL])
@pytest.mark.parametrize("seed", [0, 1])
def test_small_shapes(name, factory, seed):
    check(factory(seed))


@pytest.mark.parametrize("seed", range(10))
def test_c1_all_seeds(seed):
    check(wl.c1(seed))


@pytest.mark.parametrize("seed", range(3))
def test_c2_stochastic(seed):
    check(wl.c2_stochastic(seed))


@pytest.mark.parametrize("seed", [0, 1])
def test_c3_full_size(seed):
    """B=64, k=3, V=128256 bf16, T=0.8: the timed workload, every request checked."""
    gpu, ref, amb, dis = check(wl.c3(seed))
    assert 0 < gpu["num_accepted"].mean() < 3


def test_c3_disagreements_over_many_seeds():
    """Twelve seeds of the timed workload (768 requests, 3072 rows): requests that
    differ from the oracle stay below 1e-4 of the rows."""
    tot_rows = tot_dis = tot_amb = 0
    for seed in range(12):
        case = wl.c3(100 + seed)
        gpu = H.run_stochastic(case)
        ref = H.oracle_stochastic(case)
        amb, dis = H.compare_stochastic(gpu, ref, None, case.name)
        tot_rows += case.rows
        tot_dis += dis
        tot_amb += amb
    print(f"c3 x12: {tot_amb} ambiguous requests, {tot_dis} differ, {tot_rows} rows")
    assert tot_dis <= 1e-4 * tot_rows


@functools.lru_cache(maxsize=2)
def _c4(seed):
    return wl.c4(seed)  # 1.7 GB of logits: generated once per seed for both schedules


@pytest.mark.parametrize("seed", [0, 1])
def test_c4_full_size(seed):
    """B=256, k=5, V=151936 fp32 (the low-acceptance workload): every request
    checked against the oracle."""
    check(_c4(seed))


def test_identical_draft_accepts_everything():
    case = wl.gaussian_stochastic(3, 16, 4, 20000, "bf16", target_sd=2.0, draft_noise_sd=1.0)
    case.draft = case.target[:, :case.k, :].copy()
    gpu, ref, _, _ = check(case)
    assert np.all(gpu["num_accepted"] == case.k)


def test_disjoint_support_rejects_first():
    case = wl.gaussian_stochastic(4, 8, 3, 4096, "f32", target_sd=1.0, draft_noise_sd=1.0)
    case.target[:, :, 1::2] = -np.inf
    case.draft[:, :, 0::2] = -np.inf
    case.draft_tokens = (case.draft_tokens | 1).astype(np.int32)
    gpu, ref, _, _ = check(case)
    assert np.all(gpu["num_accepted"] == 0)
    assert np.all(gpu["out_tokens"][:, 0] % 2 == 0)


def test_out_of_range_drafts_are_rejected():
    case = wl.gaussian_stochastic(5, 4, 3, 5000, "bf16", target_sd=1.0, draft_noise_sd=0.1)
    case.draft_tokens[:, 1] = np.array([5000, -1, 1 << 30, -7], np.int32)
    case.uniforms[:] = 0.0  # tests before position 1 accept
    gpu, ref, _, _ = check(case)
    assert np.all(gpu["num_accepted"] <= 1)


def test_two_streams_with_the_default_workspace():
    """Two calls in flight at once on two streams, both with the binding's
    default workspace (one buffer per stream): both match the oracle."""
    cases = [wl.c3(31, B=16), wl.c3(32, B=16)]
    dev = torch.device("cuda", 0)
    ins = []
    for c in cases:
        ins.append((wl.to_device(c.target, c.dtype), wl.to_device(c.draft, c.dtype),
                    wl.to_device(c.draft_tokens.astype(np.int32)),
                    wl.to_device(c.uniforms.astype(np.float32))))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for c, (t, d, x, u), st in zip(cases, ins, streams):
            with torch.cuda.stream(st):
                outs.append((c, *sv.spec_verify_stochastic(t, d, x, u, c.temperature)))
    torch.cuda.synchronize()
    for c, out, acc in outs:
        gpu = dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                   p_at_draft=np.zeros((c.B, c.k)), q_at_draft=np.zeros((c.B, c.k)))
        ref = H.oracle_stochastic(c)
        ref = dict(ref, p_at_draft=np.zeros((c.B, c.k)), q_at_draft=np.zeros((c.B, c.k)))
        amb, dis = H.compare_stochastic(gpu, ref, label=c.name)
        assert dis <= 1e-4 * c.rows
    del dev


def test_repeat_calls_are_bit_identical():
    case = wl.c3(7, B=16)
    a = H.run_stochastic(case)
    b = H.run_stochastic(case)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_emitted_tokens_distributed_as_p():
    """Chi-squared on the GPU path, V=8, k=2, 10^6 trials (same law as the oracle pin)."""
    rng = np.random.default_rng(16)
    V, k, n = 8, 2, 1_000_000
    tl = rng.normal(0, 1.2, (k + 1, V)).astype(np.float32)
    dl = (tl[:k] + rng.normal(0, 1.0, (k, V))).astype(np.float32)
    p, q = lib_softmax(tl), lib_softmax(dl)
    x = np.stack([sample_from(rng, q[i], n) for i in range(k)], axis=1)
    u = rng.random((n, k + 1), dtype=np.float32)
    dev = torch.device("cuda", 0)
    t = torch.from_numpy(tl).to(dev).expand(n, k + 1, V).contiguous()
    d = torch.from_numpy(dl).to(dev).expand(n, k, V).contiguous()
    out, s = sv.spec_verify_stochastic(t, d, torch.from_numpy(x).to(dev),
                                       torch.from_numpy(u).to(dev), 1.0)
    out, s = out.cpu().numpy(), s.cpu().numpy()
    assert chi2_stat(np.bincount(out[:, 0], minlength=V), p[0]) < CHI2_DF7_P001
    assert chi2_stat(np.bincount(out[s >= 1, 1], minlength=V), p[1]) < CHI2_DF7_P001
    assert chi2_stat(np.bincount(out[s >= 2, 2], minlength=V), p[2]) < CHI2_DF7_P001


SCHEDULE_CASES = [
    lambda: wl.c3(21),
    lambda: wl.gaussian_stochastic(22, 5, 3, 40000, "bf16", target_sd=3.0, draft_noise_sd=1.0),
    lambda: wl.gaussian_stochastic(23, 3, 0, 33000, "f32", target_sd=2.0, draft_noise_sd=1.0),
    lambda: wl.gaussian_stochastic(24, 64, 5, 8, "f32", target_sd=1.0, draft_noise_sd=1.0),
    lambda: wl.c4(25, B=6),
    # small requests: a few one-vector tiles and one stop-row chunk
    lambda: wl.gaussian_stochastic(26, 4, 3, 1000, "f32", target_sd=2.0, draft_noise_sd=1.0),
    lambda: wl.gaussian_stochastic(27, 3, 2, 2048, "bf16", target_sd=3.0, draft_noise_sd=1.0),
]


@pytest.mark.parametrize("make", SCHEDULE_CASES, ids=["c3", "bf16-V40000", "k0", "V8", "c4-B6",
                                                      "f32-V1000", "bf16-V2048"])
def test_schedules_are_bit_identical(make, schedule):
    """The one-launch schedule, the two-kernel schedule, the sampling kernel
    whose workgroups compute the statistics themselves, and the one-launch
    schedule with every request's sampling right behind its statistics give the
    same bits, and leave the workspace all zero."""
    from draft_token_verification_verify_amd import _lib

    if schedule != "auto":
        pytest.skip("compares all schedules itself")
    case = make()
    ws = torch.zeros(sv.spec_verify_workspace_bytes(0, case.B, case.k + 1, case.V,
                                                    _lib.BF16 if case.dtype == "bf16" else _lib.F32),
                     dtype=torch.uint8, device="cuda")
    results = {}
    try:
        for name, code in [("auto", _lib.SCHEDULE_AUTO), ("two", _lib.SCHEDULE_TWO_KERNELS),
                           ("self", _lib.SCHEDULE_SELF_COMPUTE),
                           ("interleaved", _lib.SCHEDULE_INTERLEAVED)]:
            sv.spec_verify_set_schedule(code)
            results[name] = H.run_stochastic(case, workspace=ws)
            torch.cuda.synchronize()
            assert int(torch.count_nonzero(ws)) == 0, f"workspace not zero after {name}"
    finally:
        sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)
    for name in ("two", "self", "interleaved"):
        for key in results["auto"]:
            np.testing.assert_array_equal(results[name][key], results["auto"][key],
                                          err_msg=f"{case.name}: {name} vs auto, {key}")
    H.compare_stochastic(results["auto"], H.oracle_stochastic(case), label=case.name)
