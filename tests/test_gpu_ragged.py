"""GPU parity: per-request draft lengths (each request verified over its own
window in buffers padded to k; page "TensorRT-LLM source teardown (10)",
acceptance pipeline, step 2) against the oracle, through the ragged entry
points of the C ABI.  Same bar as the dense calls."""
import numpy as np
import pytest
import torch

import draft_token_verification_verify_amd as sv
from draft_token_verification_verify_amd import _lib
from draft_token_verification_verify_amd import workloads as wl
from tests import gpu_helpers as H
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["auto", "two-kernels", "interleaved"])
def schedule(request):
    sv.spec_verify_set_schedule({"auto": _lib.SCHEDULE_AUTO,
                                 "two-kernels": _lib.SCHEDULE_TWO_KERNELS,
                                 "interleaved": _lib.SCHEDULE_INTERLEAVED}[request.param])
    yield request.param
    sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)


def lens_for(seed, B, k):
    """Draft lengths covering 0, k, values in between and out-of-range values."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, k + 1, B).astype(np.int32)
    if B >= 4:
        lens[:4] = [0, k, -3, k + 7]
    return lens


CASES = [
    ("c3-B16", lambda s: wl.c3(s, B=16)),
    ("bf16-V40000-k5", lambda s: wl.gaussian_stochastic(s, 9, 5, 40000, "bf16", target_sd=3.0,
                                                          draft_noise_sd=0.7)),
    ("f32-V50001-k4-unaligned", lambda s: wl.gaussian_stochastic(s, 7, 4, 50001, "f32",
                                                                   target_sd=2.0,
                                                                   draft_noise_sd=0.7)),
    ("f32-V9-k6", lambda s: wl.gaussian_stochastic(s, 32, 6, 9, "f32", target_sd=1.0,
                                                     draft_noise_sd=1.0)),
    ("c4-B8", lambda s: wl.c4(s, B=8)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[n for n, _ in CASES])
@pytest.mark.parametrize("seed", [0, 1])
def test_stochastic_ragged(name, make, seed):
    case = make(seed)
    lens = lens_for(seed + 40, case.B, case.k)
    gpu = H.run_stochastic(case, draft_lens=lens)
    ref = H.oracle_stochastic(case, draft_lens=lens)
    amb, dis = H.compare_stochastic(gpu, ref, label=name)
    assert dis <= 1e-4 * case.rows
    kb = np.clip(lens, 0, case.k)
    assert np.all(gpu["num_accepted"] <= kb)
    for b in range(case.B):
        assert np.all(gpu["p_at_draft"][b, kb[b]:] == 0)


def test_ragged_full_lengths_equal_dense_call():
    case = wl.c3(5, B=12)
    dense = H.run_stochastic(case)
    ragged = H.run_stochastic(case, draft_lens=np.full(case.B, case.k, np.int32))
    for key in dense:
        np.testing.assert_array_equal(ragged[key], dense[key], err_msg=key)


def test_ragged_workspace_left_zero():
    case = wl.gaussian_stochastic(6, 10, 4, 33000, "bf16", target_sd=2.0, draft_noise_sd=1.0)
    ws = torch.zeros(sv.spec_verify_workspace_bytes(0, case.B, case.k + 1, case.V, _lib.BF16),
                     dtype=torch.uint8, device="cuda")
    for seed in range(3):
        lens = lens_for(seed, case.B, case.k)
        gpu = H.run_stochastic(case, workspace=ws, draft_lens=lens)
        H.compare_stochastic(gpu, H.oracle_stochastic(case, draft_lens=lens), label=case.name)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0


@pytest.mark.parametrize("B,k,V,dtype", [(8, 4, 32000, "bf16"), (5, 6, 77777, "bf16"),
                                         (16, 3, 4096, "f32"), (40, 5, 30, "f32")])
def test_greedy_ragged(B, k, V, dtype, schedule):
    if schedule != "auto":
        pytest.skip("greedy has one schedule")
    rng = np.random.default_rng(B + k)
    t32 = np.round(rng.normal(0, 2.0, (B, k + 1, V)) * 2).astype(np.float32) / 2
    target = wl.bf16_bits(t32) if dtype == "bf16" else t32
    tf = wl.bits_to_float(target) if dtype == "bf16" else target
    x = np.argmax(tf, axis=2)[:, :k].astype(np.int32).copy()
    x[rng.random((B, k)) < 0.2] = 0
    case = wl.GreedyCase(f"ragged-greedy-{dtype}-B{B}-k{k}-V{V}", B, k, V, dtype, target, x)
    lens = lens_for(B, B, k)
    gpu = H.run_greedy(case, draft_lens=lens)
    ref = oracle.greedy(case.target, case.draft_tokens, draft_lens=lens)
    np.testing.assert_array_equal(gpu["num_accepted"], ref["num_accepted"])
    np.testing.assert_array_equal(gpu["out_tokens"], ref["out_tokens"])
