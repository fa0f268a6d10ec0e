"""The linear calls' bounded waits, forced from the host.  With a poll limit of
0 the sampling workgroups (stochastic) and the epilogue workgroups (greedy,
tree) give up on statistics not yet published after one poll, compute what is
missing themselves and mark the workspace stale.  Results still match the
oracle; later calls on that workspace, which then compute every statistic
themselves and ignore published ones (a late publish may have left one
behind), match too; and a workspace zeroed again is back to normal and left
all zero.  Every wait ends by its limit and the fallback is the code the
self-compute schedule runs, so nothing here can hang."""
import numpy as np
import pytest
import torch

import oracle
import draft_token_verification_verify_amd as sv
from draft_token_verification_verify_amd import _lib
from draft_token_verification_verify_amd import workloads as wl
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture
def poll_limit():
    """Sets the poll limit through the testing hook; restores the default."""
    lib = _lib.load()
    yield lib.spec_verify_debug_spin_limit
    lib.spec_verify_debug_spin_limit(-1)


def _zeroed(nbytes):
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    return ws


@pytest.mark.parametrize("schedule", ["auto", "interleaved"])
def test_stochastic_gives_up_and_stays_correct(poll_limit, schedule):
    case = wl.gaussian_stochastic(31, 16, 3, 40000, "bf16", target_sd=3.0, draft_noise_sd=1.0)
    ref = H.oracle_stochastic(case)
    ws = _zeroed(sv.spec_verify_workspace_bytes(_lib.MODE_STOCHASTIC, case.B, case.k + 1,
                                                case.V, _lib.BF16))
    code = _lib.SCHEDULE_AUTO if schedule == "auto" else _lib.SCHEDULE_INTERLEAVED
    sv.spec_verify_set_schedule(code)
    try:
        poll_limit(0)
        for rep in range(3):
            gpu = H.run_stochastic(case, workspace=ws)
            amb, dis = H.compare_stochastic(gpu, ref, label=f"limit 0, call {rep}")
            assert dis <= 1e-4 * case.rows
            if rep == 0:  # a give-up leaves the stale flag set (and partials behind)
                torch.cuda.synchronize()
                assert int(torch.count_nonzero(ws)) > 0, "no wait gave up"
        poll_limit(-1)
        gpu = H.run_stochastic(case, workspace=ws)
        amb, dis = H.compare_stochastic(gpu, ref, label="default limit after give-ups")
        assert dis <= 1e-4 * case.rows
        ws.zero_()
        torch.cuda.synchronize()
        gpu = H.run_stochastic(case, workspace=ws)
        H.compare_stochastic(gpu, ref, label="zeroed workspace")
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws)) == 0, "workspace not zero after a normal call"
    finally:
        sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)


def test_greedy_gives_up_and_stays_exact(poll_limit):
    case = wl.gaussian_greedy(32, 16, 4, 40000, "bf16", target_sd=2.0, draft_noise_sd=0.5)
    ref = oracle.greedy(case.target, case.draft_tokens)
    ws = _zeroed(sv.spec_verify_workspace_bytes(_lib.MODE_GREEDY, case.B, case.k + 1, case.V,
                                                _lib.BF16))
    poll_limit(0)
    for rep in range(3):
        gpu = H.run_greedy(case, workspace=ws)
        np.testing.assert_array_equal(gpu["out_tokens"], ref["out_tokens"], f"call {rep}")
        np.testing.assert_array_equal(gpu["num_accepted"], ref["num_accepted"], f"call {rep}")
        if rep == 0:  # a give-up leaves the stale flag set (and maxima behind)
            torch.cuda.synchronize()
            assert int(torch.count_nonzero(ws)) > 0, "no wait gave up"
    poll_limit(-1)
    gpu = H.run_greedy(case, workspace=ws)
    np.testing.assert_array_equal(gpu["out_tokens"], ref["out_tokens"])
    ws.zero_()
    torch.cuda.synchronize()
    gpu = H.run_greedy(case, workspace=ws)
    np.testing.assert_array_equal(gpu["out_tokens"], ref["out_tokens"])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0, "workspace not zero after a normal call"
