"""Helpers shared by the GPU parity tests: move seeded NumPy cases to the device,
run the HIP path through the binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import draft_token_verification_verify_amd as sv
import oracle
from draft_token_verification_verify_amd.workloads import to_device as to_dev

# p(x_i), q(x_i) agreement: 1e-5 relative, with a 1e-30 absolute floor so exact
# zeros compare equal.
PROB_RTOL = 1e-5
PROB_ATOL = 1e-30
# A stochastic request is ambiguous when one of its decisions lies within this
# distance of its threshold or CDF boundary; disagreements there are counted.
GUARD = 1e-6


def run_stochastic(case, *, workspace=None, draft_lens=None):
    """Run the case through the binding (the ragged entry point when
    ``draft_lens`` is given)."""
    dev = torch.device("cuda", 0)
    t = to_dev(case.target, case.dtype)
    d = to_dev(case.draft, case.dtype) if case.k > 0 else None
    x = to_dev(case.draft_tokens.astype(np.int32)) if case.k > 0 else None
    u = to_dev(case.uniforms.astype(np.float32))
    p = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    q = torch.empty((case.B, case.k), dtype=torch.float32, device=dev)
    if draft_lens is None:
        out, acc = sv.spec_verify_stochastic(t, d, x, u, case.temperature, p_at_draft=p,
                                             q_at_draft=q, workspace=workspace)
    else:
        ln = to_dev(np.asarray(draft_lens, dtype=np.int32))
        out, acc = sv.spec_verify_stochastic_ragged(t, d, x, ln, u, case.temperature,
                                                    p_at_draft=p, q_at_draft=q,
                                                    workspace=workspace)
    torch.cuda.synchronize()
    return dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                p_at_draft=p.cpu().numpy(), q_at_draft=q.cpu().numpy())


def oracle_stochastic(case, rows=None, draft_lens=None):
    sel = slice(None) if rows is None else rows
    lens = None if draft_lens is None else np.asarray(draft_lens, dtype=np.int32)[sel]
    return oracle.stochastic(case.target[sel], case.draft[sel] if case.k > 0 else None,
                             case.draft_tokens[sel], case.uniforms[sel], case.temperature,
                             draft_lens=lens)


def compare_stochastic(gpu, ref, rows=None, label="", filter_band=None):
    """Assert parity; return (n_ambiguous, n_disagreeing_ambiguous).  With
    ``filter_band``, a request whose filter decisions lie within it of flipping
    counts as ambiguous too."""
    sel = slice(None) if rows is None else rows
    g_out, g_acc = gpu["out_tokens"][sel], gpu["num_accepted"][sel]
    g_p, g_q = gpu["p_at_draft"][sel], gpu["q_at_draft"][sel]
    if filter_band is None:
        amb = oracle.ambiguous_requests(ref["margins"], GUARD)
    else:
        amb = oracle.ambiguous_requests(ref["margins"], GUARD, ref["filter_margins"],
                                        filter_band)
    same = (g_acc == ref["num_accepted"]) & np.all(g_out == ref["out_tokens"], axis=1)
    bad = np.nonzero(~same & ~amb)[0]
    assert bad.size == 0, (
        f"{label}: {bad.size} non-ambiguous requests differ, first {bad[:5]}: "
        f"gpu {g_out[bad[:3]]} / {g_acc[bad[:3]]} vs oracle {ref['out_tokens'][bad[:3]]} / "
        f"{ref['num_accepted'][bad[:3]]}")
    np.testing.assert_allclose(g_p, ref["p_at_draft"], rtol=PROB_RTOL, atol=PROB_ATOL,
                               err_msg=f"{label}: p_at_draft")
    np.testing.assert_allclose(g_q, ref["q_at_draft"], rtol=PROB_RTOL, atol=PROB_ATOL,
                               err_msg=f"{label}: q_at_draft")
    # layout: accepted drafts, final token in [0, V), then -1
    B, k1 = g_out.shape
    for b in range(B):
        s = int(g_acc[b])
        assert 0 <= s < k1
        assert np.all(g_out[b, s + 1:] == -1)
        assert g_out[b, s] >= 0
    return int(amb.sum()), int((amb & ~same).sum())


def run_greedy(case, *, workspace=None, draft_lens=None):
    t = to_dev(case.target, case.dtype)
    x = to_dev(case.draft_tokens.astype(np.int32)) if case.k > 0 else None
    if draft_lens is None:
        out, acc = sv.spec_verify_greedy(t, x, workspace=workspace)
    else:
        ln = to_dev(np.asarray(draft_lens, dtype=np.int32))
        out, acc = sv.spec_verify_greedy_ragged(t, x, ln, workspace=workspace)
    torch.cuda.synchronize()
    return dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy())


def run_tree(case, *, workspace=None):
    t = to_dev(case.target, case.dtype)
    nt = to_dev(case.node_tokens.astype(np.int32))
    pa = to_dev(case.paths.astype(np.int32))
    out, acc, best, nodes = sv.spec_verify_tree(t, nt, pa, workspace=workspace)
    torch.cuda.synchronize()
    return dict(out_tokens=out.cpu().numpy(), num_accepted=acc.cpu().numpy(),
                best_path=best.cpu().numpy(), accepted_nodes=nodes.cpu().numpy())
