"""GPU parity: stochastic verification with counter-based uniforms (Philox4x64-10
draws from a per-call seed and offset; page "TensorRT-LLM source teardown (10)",
"Rejection sampling") against the oracle fed the oracle's own Philox draws."""
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


@pytest.fixture(autouse=True, params=["auto", "two-kernels", "interleaved"])
def schedule(request):
    sv.spec_verify_set_schedule({"auto": _lib.SCHEDULE_AUTO,
                                 "two-kernels": _lib.SCHEDULE_TWO_KERNELS,
                                 "interleaved": _lib.SCHEDULE_INTERLEAVED}[request.param])
    yield request.param
    sv.spec_verify_set_schedule(_lib.SCHEDULE_AUTO)


def run_philox(case, seed, offset, draft_lens=None):
    t = wl.to_device(case.target, case.dtype)
    d = wl.to_device(case.draft, case.dtype) if case.k > 0 else None
    x = wl.to_device(case.draft_tokens.astype(np.int32)) if case.k > 0 else None
    ln = None if draft_lens is None else wl.to_device(np.asarray(draft_lens, np.int32))
    dev = t.device
    p = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    q = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    out, acc = sv.spec_verify_stochastic_philox(t, d, x, ln, seed, offset, case.temperature,
                                                p_at_draft=p, q_at_draft=q)
    torch.cuda.synchronize()
    return dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                p_at_draft=p.cpu().numpy(), q_at_draft=q.cpu().numpy())


def oracle_philox(case, seed, offset, draft_lens=None):
    u = oracle.philox_uniforms(seed, offset, case.B, case.k + 1)
    return oracle.stochastic(case.target, case.draft if case.k > 0 else None, case.draft_tokens,
                             u, case.temperature, draft_lens=draft_lens)


CASES = [
    ("c3-B32", lambda: wl.c3(3, B=32)),
    ("bf16-V40000-k5", lambda: wl.gaussian_stochastic(4, 9, 5, 40000, "bf16", target_sd=3.0,
                                                        draft_noise_sd=0.7)),
    ("f32-V50001-k2-unaligned", lambda: wl.gaussian_stochastic(5, 6, 2, 50001, "f32",
                                                                 target_sd=2.0,
                                                                 draft_noise_sd=0.7)),
    ("f32-V33000-k0", lambda: wl.gaussian_stochastic(6, 5, 0, 33000, "f32", target_sd=2.0,
                                                       draft_noise_sd=1.0)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[n for n, _ in CASES])
@pytest.mark.parametrize("seed,offset", [(0, 0), (2**64 - 1, 12345), (0x9E3779B9, 2**40 + 7)])
def test_philox_matches_oracle(name, make, seed, offset):
    case = make()
    gpu = run_philox(case, seed, offset)
    ref = oracle_philox(case, seed, offset)
    amb, dis = H.compare_stochastic(gpu, ref, label=f"{name} seed {seed} offset {offset}")
    assert dis <= 1e-4 * case.rows


def test_philox_with_ragged_lengths():
    case = wl.c3(8, B=24)
    lens = np.random.default_rng(8).integers(-1, case.k + 2, case.B).astype(np.int32)
    gpu = run_philox(case, 31, 4, draft_lens=lens)
    ref = oracle_philox(case, 31, 4, draft_lens=lens)
    amb, dis = H.compare_stochastic(gpu, ref, label="philox ragged")
    assert dis <= 1e-4 * case.rows


def test_philox_offsets_give_fresh_draws_and_repeat_exactly():
    case = wl.c3(9, B=64)
    a = run_philox(case, 5, 100)
    b = run_philox(case, 5, 100)
    c = run_philox(case, 5, 101)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    assert np.any(a["out_tokens"] != c["out_tokens"])


def test_philox_emitted_tokens_distributed_as_p():
    """Chi-squared, V=8, k=2, 10^6 requests whose uniforms are all Philox draws."""
    rng = np.random.default_rng(46)
    V, k, n = 8, 2, 1_000_000
    tl = rng.normal(0, 1.2, (k + 1, V)).astype(np.float32)
    dl = (tl[:k] + rng.normal(0, 1.0, (k, V))).astype(np.float32)
    p, q = lib_softmax(tl), lib_softmax(dl)
    x = np.stack([sample_from(rng, q[i], n) for i in range(k)], axis=1)
    dev = torch.device("cuda", 0)
    t = torch.from_numpy(tl).to(dev).expand(n, k + 1, V).contiguous()
    d = torch.from_numpy(dl).to(dev).expand(n, k, V).contiguous()
    out, s = sv.spec_verify_stochastic_philox(t, d, torch.from_numpy(x).to(dev), None, 2024, 7,
                                              1.0)
    out, s = out.cpu().numpy(), s.cpu().numpy()
    assert chi2_stat(np.bincount(out[:, 0], minlength=V), p[0]) < CHI2_DF7_P001
    assert chi2_stat(np.bincount(out[s >= 1, 1], minlength=V), p[1]) < CHI2_DF7_P001
    assert chi2_stat(np.bincount(out[s >= 2, 2], minlength=V), p[2]) < CHI2_DF7_P001
