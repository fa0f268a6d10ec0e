"""Checks that pin the CPU oracle to facts fixed outside the oracle itself.

Each ``check_*`` function takes an oracle library handle (``None`` = the
default build) and raises ``AssertionError`` when the oracle disagrees with a
value the pages print, a closed form, a library routine applied to a special
case, a statistical law of the method, or a brute-force enumeration.  The same
functions run against deliberately broken builds of the oracle (planted
mistakes) to show that each plausible mistake is caught by at least one check.

Sources (page title, section):
  * "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
    "Speculative Decoding": accept when p >= q, else with probability p/q; stop
    at the first rejection; residual max(0, p - q) normalised; bonus from the
    extra row; the output is distributed as sampling from p.
  * "02. Speculative Decoding" (vLLM learning book), section 2 flowchart and
    section 3 (q == p gives acceptance rate 1).
  * "TensorRT-LLM source teardown (10): speculative decoding", "MTP mechanism
    background" (the "Generation phase 1" worked example) and "Rejection
    sampling" (output layout, -1 padding).
  * "Kestrel_VLLM - 32", section 3.3: every emitted token is on the target's
    argmax chain, whatever the drafts.
  * "05 - TensorRT-LLM speculative decoding and auto-deploy": paths table.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CHI2_DF7_P001 = 24.322  # chi-squared critical value, 7 degrees of freedom, p = 0.001


# ---- independent helpers (library routines, never the oracle) -----------------

def lib_softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """torch.softmax in float64 over the last axis."""
    t = torch.from_numpy(np.asarray(logits, dtype=np.float64) / temperature)
    return torch.softmax(t, dim=-1).numpy()


def lib_inverse_cdf(weights: np.ndarray, u: float):
    """(token, distance of u*Z to the nearest CDF edge relative to Z) by searchsorted."""
    c = np.cumsum(weights)
    z = c[-1]
    j = int(np.searchsorted(c, u * z, side="right"))
    j = min(j, len(weights) - 1)
    edges = np.concatenate([[0.0], c])
    dist = np.min(np.abs(edges - u * z)) / z
    return j, dist


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def chi2_stat(counts: np.ndarray, probs: np.ndarray) -> float:
    n = counts.sum()
    expected = n * probs
    keep = expected > 0
    assert np.all(counts[~keep] == 0), "token with zero probability was emitted"
    return float(np.sum((counts[keep] - expected[keep]) ** 2 / expected[keep]))


def sample_from(rng, probs: np.ndarray, n: int) -> np.ndarray:
    return rng.choice(len(probs), size=n, p=probs / probs.sum()).astype(np.int32)


# ---- stochastic mode -------------------------------------------------------------

def check_softmax_vs_library(lib):
    """p_i(x_i), q_i(x_i) equal torch.softmax(logits / T) in float64 (f32 and bf16 inputs)."""
    rng = np.random.default_rng(11)
    for dtype in ("f32", "bf16"):
        for T in (1.0, 0.7, 1.9):
            B, k, V = 3, 2, 37
            t = rng.normal(0, 2.5, (B, k + 1, V)).astype(np.float32)
            d = rng.normal(0, 2.5, (B, k, V)).astype(np.float32)
            if dtype == "bf16":
                t, d = to_bf16_bits(t), to_bf16_bits(d)
                tf, df = bf16_bits_to_f64(t), bf16_bits_to_f64(d)
            else:
                tf, df = t.astype(np.float64), d.astype(np.float64)
            x = rng.integers(0, V, (B, k)).astype(np.int32)
            u = np.full((B, k + 1), 0.999, np.float32)
            r = oracle.stochastic(t, d, x, u, T, lib=lib)
            pt = lib_softmax(tf[:, :k, :], T)
            pd = lib_softmax(df, T)
            want_p = np.take_along_axis(pt, x[..., None], axis=2)[..., 0]
            want_q = np.take_along_axis(pd, x[..., None], axis=2)[..., 0]
            np.testing.assert_allclose(r["p_at_draft"], want_p, rtol=1e-12, atol=0)
            np.testing.assert_allclose(r["q_at_draft"], want_q, rtol=1e-12, atol=0)


def check_identical_draft_accepts_all(lib):
    """q == p: every draft accepted (acceptance rate 1), bonus = inverse CDF of p_k at u_k."""
    rng = np.random.default_rng(12)
    B, k, V, T = 64, 3, 50, 0.8
    t = rng.normal(0, 2.0, (B, k + 1, V)).astype(np.float32)
    d = t[:, :k, :].copy()
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    r = oracle.stochastic(t, d, x, u, T, lib=lib)
    assert np.all(r["num_accepted"] == k)
    np.testing.assert_array_equal(r["out_tokens"][:, :k], x)
    pk = lib_softmax(t[:, k, :], T)
    checked = 0
    for b in range(B):
        j, dist = lib_inverse_cdf(pk[b], float(u[b, k]))
        if dist < 1e-9:
            continue
        assert r["out_tokens"][b, k] == j, (b, r["out_tokens"][b, k], j)
        checked += 1
    assert checked > B // 2


def check_disjoint_support_rejects_first(lib):
    """Disjoint supports: test 0 rejects (p(x) = 0) and the token is drawn from p_0."""
    rng = np.random.default_rng(13)
    B, k, V = 200, 2, 16
    t = rng.normal(0, 1.5, (B, k + 1, V)).astype(np.float32)
    d = rng.normal(0, 1.5, (B, k, V)).astype(np.float32)
    t[:, :, 1::2] = -np.inf  # target lives on even ids
    d[:, :, 0::2] = -np.inf  # draft lives on odd ids
    x = (2 * rng.integers(0, V // 2, (B, k)) + 1).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    r = oracle.stochastic(t, d, x, u, 1.0, lib=lib)
    assert np.all(r["num_accepted"] == 0)
    assert np.all(r["out_tokens"][:, 1:] == -1)
    p0 = lib_softmax(t[:, 0, :])
    for b in range(B):
        j, dist = lib_inverse_cdf(p0[b], float(u[b, k]))
        if dist < 1e-9:
            continue
        assert r["out_tokens"][b, 0] == j
    assert np.all(r["out_tokens"][:, 0] % 2 == 0)


def check_one_hot_draft_closed_form(lib):
    """q one-hot at x: accept iff u < p(x); the residual is p with x removed."""
    rng = np.random.default_rng(14)
    B, k, V = 3000, 1, 6
    t = rng.normal(0, 1.0, (B, k + 1, V)).astype(np.float32)
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    d = np.full((B, k, V), -np.inf, np.float32)
    d[np.arange(B), 0, x[:, 0]] = 0.0
    u = rng.random((B, k + 1), dtype=np.float32)
    r = oracle.stochastic(t, d, x, u, 1.0, lib=lib)
    p0 = lib_softmax(t[:, 0, :])
    p1 = lib_softmax(t[:, 1, :])
    n_acc = n_rej = 0
    for b in range(B):
        px = p0[b, x[b, 0]]
        if abs(float(u[b, 0]) - px) < 1e-9:
            continue
        want_accept = float(u[b, 0]) < px
        assert r["num_accepted"][b] == (1 if want_accept else 0), b
        if want_accept:
            j, dist = lib_inverse_cdf(p1[b], float(u[b, 1]))
            n_acc += 1
        else:
            w = p0[b].copy()
            w[x[b, 0]] = 0.0
            j, dist = lib_inverse_cdf(w, float(u[b, 1]))
            n_rej += 1
        if dist > 1e-9:
            slot = 1 if want_accept else 0
            assert r["out_tokens"][b, slot] == j, (b, want_accept)
    assert n_acc > 100 and n_rej > 100


def check_strict_threshold(lib):
    """u equal to p/q rejects (strict '<'); the next float below accepts; p == q accepts."""
    V = 4
    t = np.array([[[0, 0, -np.inf, -np.inf], [0, 1, 2, 3]]], np.float32)  # p0 = [.5,.5,0,0]
    d = np.array([[[0, -np.inf, -np.inf, -np.inf]]], np.float32)          # q0 = [1,0,0,0]
    x = np.array([[0]], np.int32)  # P = 0.5, Q = 1: threshold exactly 0.5
    half = np.float32(0.5)
    below = np.nextafter(half, np.float32(0))
    r = oracle.stochastic(t, d, x, np.array([[half, 0.3]], np.float32), 1.0, lib=lib)
    assert r["num_accepted"][0] == 0
    assert r["out_tokens"][0, 0] == 1  # residual max(0, p - q) = [0, .5, 0, 0]
    r = oracle.stochastic(t, d, x, np.array([[below, 0.3]], np.float32), 1.0, lib=lib)
    assert r["num_accepted"][0] == 1
    # p == q exactly (identical rows): accepted whatever the uniform.
    d_same = t[:, :1, :].copy()
    r = oracle.stochastic(t, d_same, x, np.array([[np.float32(0.99999994), 0.0]], np.float32),
                          1.0, lib=lib)
    assert r["num_accepted"][0] == 1
    assert r["out_tokens"][0, 1] == 0  # u = 0 on the bonus row: first positive-weight token
    del V


def check_acceptance_frequency(lib):
    """With x ~ q and u ~ U(0,1), test 0 accepts with probability sum_x min(p(x), q(x))."""
    rng = np.random.default_rng(15)
    B, V = 200_000, 10
    tl = rng.normal(0, 1.5, V).astype(np.float32)
    dl = rng.normal(0, 1.5, V).astype(np.float32)
    p = lib_softmax(tl)
    q = lib_softmax(dl)
    t = np.broadcast_to(tl, (B, 2, V)).copy()
    d = np.broadcast_to(dl, (B, 1, V)).copy()
    x = sample_from(rng, q, B).reshape(B, 1)
    u = rng.random((B, 2), dtype=np.float32)
    r = oracle.stochastic(t, d, x, u, 1.0, lib=lib)
    alpha = float(np.minimum(p, q).sum())
    rate = float(np.mean(r["num_accepted"] == 1))
    sigma = np.sqrt(alpha * (1 - alpha) / B)
    assert abs(rate - alpha) < 5 * sigma, (rate, alpha, sigma)


def check_emitted_tokens_distributed_as_p(lib, trials: int = 1_000_000):
    """Chi-squared, V=8, k=2: 1st emitted token ~ p_0; 2nd given s>=1 ~ p_1; bonus ~ p_2."""
    rng = np.random.default_rng(16)
    V, k = 8, 2
    tl = rng.normal(0, 1.2, (k + 1, V)).astype(np.float32)
    dl = (tl[:k] + rng.normal(0, 1.0, (k, V))).astype(np.float32)
    p = lib_softmax(tl)
    q = lib_softmax(dl)
    t = np.broadcast_to(tl, (trials, k + 1, V)).copy()
    d = np.broadcast_to(dl, (trials, k, V)).copy()
    x = np.stack([sample_from(rng, q[i], trials) for i in range(k)], axis=1)
    u = rng.random((trials, k + 1), dtype=np.float32)
    r = oracle.stochastic(t, d, x, u, 1.0, lib=lib)
    out, s = r["out_tokens"], r["num_accepted"]
    first = np.bincount(out[:, 0], minlength=V)
    assert chi2_stat(first, p[0]) < CHI2_DF7_P001, ("first token", first)
    second = np.bincount(out[s >= 1, 1], minlength=V)
    assert chi2_stat(second, p[1]) < CHI2_DF7_P001, ("second token", second)
    third = np.bincount(out[s >= 2, 2], minlength=V)
    assert third.sum() > 10_000
    assert chi2_stat(third, p[2]) < CHI2_DF7_P001, ("bonus token", third)


def check_inverse_cdf_zero_weights(lib):
    """k = 0 (plain sampling of row 0) equals searchsorted(cumsum(p), u*Z, 'right')."""
    rng = np.random.default_rng(17)
    B, V = 500, 16
    t = rng.normal(0, 1.0, (B, 1, V)).astype(np.float32)
    mask = rng.random((B, V)) < 0.4
    mask[:, 0] = True  # token 0 always has zero weight
    mask[np.arange(B), rng.integers(1, V, B)] = False  # keep at least one token
    t[:, 0, :][mask] = -np.inf
    u = rng.random((B, 1), dtype=np.float32)
    u[:50] = 0.0
    r = oracle.stochastic(t, None, np.zeros((B, 0), np.int32), u, 1.0, lib=lib)
    p = lib_softmax(t[:, 0, :])
    assert np.all(r["num_accepted"] == 0)
    for b in range(B):
        if u[b, 0] == 0.0:
            assert r["out_tokens"][b, 0] == int(np.argmax(p[b] > 0)), b
            continue
        j, dist = lib_inverse_cdf(p[b], float(u[b, 0]))
        if dist > 1e-9:
            assert r["out_tokens"][b, 0] == j, b


def check_out_of_range_draft_rejected(lib):
    """A draft id outside [0, V) is rejected with P = Q = 0 reported."""
    rng = np.random.default_rng(18)
    B, k, V = 4, 3, 9
    t = rng.normal(0, 1.0, (B, k + 1, V)).astype(np.float32)
    d = t[:, :k, :].copy()
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    x[:, 1] = np.array([V, -1, V + 100, -7], np.int32)
    u = np.full((B, k + 1), 0.5, np.float32)
    r = oracle.stochastic(t, d, x, u, 1.0, lib=lib)
    assert np.all(r["num_accepted"] == 1)
    assert np.all(r["p_at_draft"][:, 1] == 0) and np.all(r["q_at_draft"][:, 1] == 0)


# ---- the worked example ------------------------------------------------------------

def load_fgxy():
    spec = {}
    with open(os.path.join(GOLDEN, "fgxy_greedy.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            spec[key] = vals
    ids = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in spec["tokens"]}
    ids["-1"] = -1
    return dict(
        V=int(spec["vocab"][0]),
        drafts=[ids[v] for v in spec["drafts"]],
        rows=[ids[v] for v in spec["target_row_tokens"]],
        out=[ids[v] for v in spec["expected_out"]],
        accepted=int(spec["expected_num_accepted"][0]),
    )


def check_fgxy_worked_example(lib):
    """Greedy on the printed example gives F G X -1, two accepted; so does sampling with
    one-hot target rows (the target's own token at each row), for any uniforms."""
    ex = load_fgxy()
    V, k = ex["V"], len(ex["drafts"])
    t = np.zeros((1, k + 1, V), np.float32)
    for i, tok in enumerate(ex["rows"]):
        t[0, i, tok] = 5.0
    x = np.array([ex["drafts"]], np.int32)
    g = oracle.greedy(t, x, lib=lib)
    assert g["out_tokens"][0].tolist() == ex["out"]
    assert g["num_accepted"][0] == ex["accepted"]
    t1 = np.full((1, k + 1, V), -np.inf, np.float32)
    for i, tok in enumerate(ex["rows"]):
        t1[0, i, tok] = 0.0
    rng = np.random.default_rng(19)
    for _ in range(20):
        d = rng.normal(0, 1.0, (1, k, V)).astype(np.float32)
        u = rng.random((1, k + 1), dtype=np.float32)
        s = oracle.stochastic(t1, d, x, u, 1.0, lib=lib)
        assert s["out_tokens"][0].tolist() == ex["out"]
        assert s["num_accepted"][0] == ex["accepted"]


# ---- greedy mode -------------------------------------------------------------------

def check_greedy_argmax_chain(lib):
    """Emitted tokens are the target's argmax chain (np.argmax, first maximum), whatever
    the drafts; the count is the number of leading matches; -1 after the last token."""
    rng = np.random.default_rng(20)
    for k in (0, 1, 3, 8):
        B, V = 40, 300
        t32 = np.round(rng.normal(0, 2.0, (B, k + 1, V)) * 2) / 2  # many ties
        t = to_bf16_bits(t32.astype(np.float32))
        tf = bf16_bits_to_f64(t)
        a = np.argmax(tf, axis=2)
        x = a[:, :k].astype(np.int32).copy()
        corrupt = rng.random((B, k)) < 0.25
        x[corrupt] = rng.integers(0, V, int(corrupt.sum()))
        x[0, :] = (a[0, :k] + 1) % V  # a request with zero accepted drafts
        r = oracle.greedy(t, x, lib=lib)
        for b in range(B):
            s = 0
            while s < k and x[b, s] == a[b, s]:
                s += 1
            assert r["num_accepted"][b] == s
            assert r["out_tokens"][b, :s + 1].tolist() == a[b, :s + 1].tolist()
            assert np.all(r["out_tokens"][b, s + 1:] == -1)
        np.testing.assert_array_equal(r["argmax"], a)


# ---- tree mode ---------------------------------------------------------------------

def _tree_bruteforce(a, tok, paths, N):
    """Best (m, lowest row) by enumerating path rows; a node counts when its token is
    the argmax of the row of the entry before it on that path."""
    best_m, best_row = -1, -1
    for row_idx, row in enumerate(paths):
        if not (0 <= row[0] <= N):
            continue
        good = []
        for t in range(1, len(row)):
            child = row[t]
            if not (0 <= child <= N):
                break
            good.append(tok[child] == a[row[t - 1]])
        m = 0
        for g in good:
            if not g:
                break
            m += 1
        if m > best_m:
            best_m, best_row = m, row_idx
    return best_m, best_row


def check_tree_bruteforce(lib):
    """Tiny trees (N <= 7, V <= 3): the deepest accepted root-to-node chain over all
    nodes equals num_accepted; the chosen row is the lowest row reaching it."""
    from draft_token_verification_verify_amd.workloads import _paths_of, _random_tree

    rng = np.random.default_rng(21)
    for trial in range(300):
        N = int(rng.integers(1, 8))
        depth = int(rng.integers(1, N + 1))
        V = int(rng.integers(1, 4))
        par = _random_tree(rng, N, depth, max_children=10)
        L = depth + 1
        P = N
        paths = _paths_of(par, P, L)
        t = rng.integers(0, 3, (1, N + 1, V)).astype(np.float32)
        a = np.argmax(t[0].astype(np.float64), axis=1)
        tok = rng.integers(0, V, N + 1).astype(np.int32)
        r = oracle.tree(t, tok[None], paths[None], lib=lib)
        # deepest accepted chain over every node of the tree
        depth_ok = np.full(N + 1, -1)
        depth_ok[0] = 0
        for n in range(1, N + 1):  # BFS numbering: parents come first
            pn = par[n]
            if depth_ok[pn] >= 0 and tok[n] == a[pn]:
                depth_ok[n] = depth_ok[pn] + 1
        want_m = int(depth_ok.max())
        m, row = _tree_bruteforce(a, tok, paths, N)
        assert m == want_m, (trial, m, want_m)
        assert r["num_accepted"][0] == want_m, trial
        assert r["best_path"][0] == row, trial
        chain = paths[row, : want_m + 1]
        want_out = [int(tok[n]) for n in chain[1:]] + [int(a[chain[-1]])]
        want_out += [-1] * (L - len(want_out))
        assert r["out_tokens"][0].tolist() == want_out, trial
        want_nodes = list(chain[1:]) + [-1] * (L - want_m)
        assert r["accepted_nodes"][0].tolist() == want_nodes, trial


def check_chain_tree_equals_greedy(lib):
    """A tree that is a single chain gives the greedy result on the same rows."""
    rng = np.random.default_rng(22)
    B, k, V = 16, 5, 50
    t = rng.normal(0, 2, (B, k + 1, V)).astype(np.float32)
    a = np.argmax(t, axis=2)
    x = a[:, :k].astype(np.int32).copy()
    flip = rng.random((B, k)) < 0.2
    x[flip] = (x[flip] + 1) % V
    g = oracle.greedy(t, x, lib=lib)
    tok = np.concatenate([np.zeros((B, 1), np.int32), x], axis=1)
    paths = np.full((B, 3, k + 1), -1, np.int32)
    paths[:, 1, :] = np.arange(k + 1)
    r = oracle.tree(t, tok, paths, lib=lib)
    np.testing.assert_array_equal(r["num_accepted"], g["num_accepted"])
    np.testing.assert_array_equal(r["out_tokens"], g["out_tokens"])
    assert np.all(r["best_path"] == 1)


def check_tree_unused_rows(lib):
    """No usable row: emit the root's argmax; out-of-range entries end a path."""
    V, N, L = 5, 3, 4
    t = np.zeros((1, N + 1, V), np.float32)
    for n, j in enumerate([2, 3, 4, 1]):
        t[0, n, j] = 1.0
    tok = np.array([[0, 2, 3, 4]], np.int32)  # the chain 0-1-2-3 is fully accepted
    paths = np.full((1, 2, L), -1, np.int32)
    r = oracle.tree(t, tok, paths, lib=lib)
    assert r["out_tokens"][0].tolist() == [2, -1, -1, -1]
    assert r["num_accepted"][0] == 0 and r["best_path"][0] == -1
    paths[0, 0] = [0, 1, 9, 3]  # 9 is not a node: the path ends after node 1
    paths[0, 1] = [0, 1, 2, 3]
    r = oracle.tree(t, tok, paths, lib=lib)
    assert r["num_accepted"][0] == 3 and r["best_path"][0] == 1
    assert r["out_tokens"][0].tolist() == [2, 3, 4, 1]
    paths[0, 1] = [0, 1, 2, -1]
    r = oracle.tree(t, tok, paths, lib=lib)
    assert r["num_accepted"][0] == 2 and r["out_tokens"][0].tolist() == [2, 3, 4, -1]


# ---- per-request draft lengths -----------------------------------------------------
# Page "TensorRT-LLM source teardown (10)", acceptance-pipeline step 2: with
# ragged verification each request is verified over its own window while the
# buffers stay padded to the static maximum; padding must never count.

def _ragged_case(rng, B, k, V, dtype):
    t = rng.normal(0, 1.5, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rng.normal(0, 1.0, (B, k, V))).astype(np.float32)
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    # drafts often equal to the target's favourite token, so tests accept
    fav = rng.random((B, k)) < 0.5
    x[fav] = np.argmax(t[:, :k], axis=2)[fav]
    u = rng.random((B, k + 1), dtype=np.float32)
    if dtype == "bf16":
        t, d = to_bf16_bits(t), to_bf16_bits(d)
    return t, d, x, u


def check_ragged_is_each_request_alone(lib):
    """Request b with draft length k_b (clamped to [0, k]) gives what a request of
    length k_b gives on its own: first k_b + 1 target rows, first k_b draft rows and
    drafts, uniforms 0..k_b; the padded slots read -1 (tokens) and 0 (P, Q)."""
    rng = np.random.default_rng(31)
    B, k, V, T = 24, 4, 40, 0.9
    for dtype in ("f32", "bf16"):
        t, d, x, u = _ragged_case(rng, B, k, V, dtype)
        lens = rng.integers(-2, k + 3, B).astype(np.int32)
        r = oracle.stochastic(t, d, x, u, T, draft_lens=lens, lib=lib)
        for b in range(B):
            kb = int(min(max(lens[b], 0), k))
            sl = slice(b, b + 1)
            alone = oracle.stochastic(t[sl, :kb + 1], d[sl, :kb] if kb else None, x[sl, :kb],
                                      u[sl, :kb + 1], T, lib=lib)
            assert r["num_accepted"][b] == alone["num_accepted"][0]
            assert np.array_equal(r["out_tokens"][b, :kb + 1], alone["out_tokens"][0])
            assert np.all(r["out_tokens"][b, kb + 1:] == -1)
            assert np.array_equal(r["p_at_draft"][b, :kb], alone["p_at_draft"][0])
            assert np.all(r["p_at_draft"][b, kb:] == 0) and np.all(r["q_at_draft"][b, kb:] == 0)
        # every draft length at k: the padded call is the plain call
        full = oracle.stochastic(t, d, x, u, T, draft_lens=np.full(B, k, np.int32), lib=lib)
        plain = oracle.stochastic(t, d, x, u, T, lib=lib)
        for key in ("out_tokens", "num_accepted", "p_at_draft", "q_at_draft"):
            assert np.array_equal(full[key], plain[key]), key


def check_ragged_zero_length_samples_row_zero(lib):
    """Draft length 0: no test; the token is the inverse-CDF draw of softmax(row 0 / T)
    at uniforms[b, 0] (library softmax and searchsorted), then -1 padding."""
    rng = np.random.default_rng(32)
    B, k, V, T = 64, 3, 12, 0.7
    t, d, x, u = _ragged_case(rng, B, k, V, "f32")
    r = oracle.stochastic(t, d, x, u, T, draft_lens=np.zeros(B, np.int32), lib=lib)
    p0 = lib_softmax(t[:, 0], T)
    assert np.all(r["num_accepted"] == 0)
    assert np.all(r["out_tokens"][:, 1:] == -1)
    for b in range(B):
        j, _ = lib_inverse_cdf(p0[b], float(u[b, 0]))
        assert r["out_tokens"][b, 0] == j, b


def check_greedy_ragged(lib):
    """Greedy with draft length k_b: leading matches against np.argmax over rows
    0..k_b-1 only, then the argmax of row s; -1 after it."""
    rng = np.random.default_rng(33)
    B, k, V = 40, 5, 30
    t = np.round(rng.normal(0, 2, (B, k + 1, V))).astype(np.float32)
    a = np.argmax(t, axis=2)
    x = a[:, :k].astype(np.int32).copy()
    x[rng.random((B, k)) < 0.15] = 0
    lens = rng.integers(0, k + 1, B).astype(np.int32)
    r = oracle.greedy(t, x, draft_lens=lens, lib=lib)
    for b in range(B):
        kb = int(lens[b])
        s = 0
        while s < kb and x[b, s] == a[b, s]:
            s += 1
        assert r["num_accepted"][b] == s
        want = list(x[b, :s]) + [a[b, s]] + [-1] * (k - s)
        assert list(r["out_tokens"][b]) == want, b


# ---- counter-based uniforms ------------------------------------------------------
# Page "TensorRT-LLM source teardown (10)", "Rejection sampling": uniforms come
# from Philox with a per-call (seed, offset).  The generator is Philox4x64-10;
# NumPy's Philox bit generator is the same published generator and serves as
# the library pin.

def numpy_philox_block(counter, key) -> np.ndarray:
    """Philox4x64-10 block at `counter` by NumPy.  NumPy's Philox advances its
    256-bit little-endian counter before producing a block, so it is started one
    below."""
    n = sum(int(v) << (64 * i) for i, v in enumerate(counter)) - 1
    n %= 1 << 256
    prev = np.array([(n >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.asarray(key, dtype=np.uint64), counter=prev)
    return bg.random_raw(4)


def check_philox_matches_numpy(lib):
    """oracle Philox4x64-10 blocks equal NumPy's on random and edge counters/keys."""
    rng = np.random.default_rng(41)
    cases = [([0, 0, 0, 0], [0, 0]), ([0, 1, 0, 0], [1, 0]),
             ([2**64 - 1, 2**64 - 1, 3, 0], [2**64 - 1, 2**64 - 1])]
    for _ in range(20):
        cases.append((rng.integers(0, 2**64 - 1, 4, dtype=np.uint64, endpoint=True),
                      rng.integers(0, 2**64 - 1, 2, dtype=np.uint64, endpoint=True)))
    for c, k in cases:
        got = oracle.philox4x64_10(np.array(c, np.uint64), np.array(k, np.uint64), lib=lib)
        assert np.array_equal(got, numpy_philox_block(c, k)), (c, k)


def check_philox_uniform_layout(lib):
    """uniforms[b, i] = top 24 bits of word i % 4 of the block at counter
    (offset, b, i // 4, 0), key (seed, 0), times 2^-24; in [0, 1), mean 1/2."""
    seed, offset, B, n = 0x1234_5678_9ABC_DEF0, 77, 5, 11
    u = oracle.philox_uniforms(seed, offset, B, n, lib=lib)
    for b in range(B):
        for i in range(n):
            w = numpy_philox_block([offset, b, i // 4, 0], [seed, 0])[i % 4]
            assert u[b, i] == np.float32(float(int(w) >> 40) * 2.0**-24), (b, i)
    big = oracle.philox_uniforms(9, 3, 2000, 50, lib=lib)
    assert big.min() >= 0.0 and big.max() < 1.0
    assert abs(float(big.mean()) - 0.5) < 5 * np.sqrt(1 / 12 / big.size)


# ---- symmetric filtering ------------------------------------------------------------
# Page "TensorRT-LLM source teardown (10)", "Rejection sampling": temperature,
# top-k, top-p and min_p must filter target and draft identically.  Readings:
# thresholds on the logit; top-k keeps ties of the k-th value; top-p keeps the
# smallest run of the top-k survivors (descending) whose renormalised mass
# reaches top_p; min_p keeps p >= min_p * max p; in that order.

def _one_row_case(logits_t, logits_d, token):
    t = np.array([[logits_t, logits_t]], np.float32)  # k = 1: row 0 tested, row 1 bonus
    d = np.array([[logits_d]], np.float32)
    x = np.array([[token]], np.int32)
    u = np.array([[0.5, 0.5]], np.float32)
    return t, d, x, u


def check_filter_off_is_plain(lib):
    """top_k in {0, V, V+3}, top_p = 1, min_p = 0 give the unfiltered results."""
    rng = np.random.default_rng(51)
    B, k, V = 16, 3, 20
    t = rng.normal(0, 1.5, (B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rng.normal(0, 1, (B, k, V))).astype(np.float32)
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    plain = oracle.stochastic(t, d, x, u, 0.9, lib=lib)
    for tk in (V, V + 3):
        r = oracle.stochastic(t, d, x, u, 0.9, top_k=tk, lib=lib)
        for key in ("out_tokens", "num_accepted", "p_at_draft", "q_at_draft"):
            assert np.array_equal(r[key], plain[key]), (tk, key)


def check_top_k_closed_form(lib):
    """top-k: P = p(x) / sum of the k largest p (torch.topk), 0 outside them; the
    k-th value's ties are all kept."""
    rng = np.random.default_rng(52)
    V = 12
    logits = rng.normal(0, 2, V).astype(np.float32)
    p = lib_softmax(logits)
    for kk in (1, 3, 7):
        top = torch.topk(torch.from_numpy(p), kk).indices.numpy()
        for token in range(V):
            t, d, x, u = _one_row_case(logits, logits, token)
            r = oracle.stochastic(t, d, x, u, 1.0, top_k=kk, lib=lib)
            want = p[token] / p[top].sum() if token in top else 0.0
            assert abs(r["p_at_draft"][0, 0] - want) < 1e-12, (kk, token)
    tied = np.array([2, 1, 1, 0], np.float32)
    t, d, x, u = _one_row_case(tied, tied, 2)
    r = oracle.stochastic(t, d, x, u, 1.0, top_k=2, lib=lib)
    e = np.exp([2.0, 1.0, 1.0])
    assert abs(r["p_at_draft"][0, 0] - e[1] / e.sum()) < 1e-12


def check_top_p_closed_form(lib):
    """top-p on p = (.5, .3, .2): 0.45 keeps {0}; 0.75 keeps {0, 1}; 0.85 keeps all.
    top-k = 3 then top-p = 0.75 on p = (.4, .3, .2, .1) renormalises first and keeps
    {0, 1} (without renormalising it would keep {0, 1, 2})."""
    base = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32)
    p = lib_softmax(base)
    for top_p, kept in ((0.45, [0]), (0.75, [0, 1]), (0.85, [0, 1, 2])):
        for token in range(3):
            t, d, x, u = _one_row_case(base, base, token)
            r = oracle.stochastic(t, d, x, u, 1.0, top_p=top_p, lib=lib)
            want = p[token] / p[kept].sum() if token in kept else 0.0
            assert abs(r["p_at_draft"][0, 0] - want) < 1e-9, (top_p, token)
    four = np.log(np.array([0.4, 0.3, 0.2, 0.1])).astype(np.float32)
    p4 = lib_softmax(four)
    for token in range(4):
        t, d, x, u = _one_row_case(four, four, token)
        r = oracle.stochastic(t, d, x, u, 1.0, top_k=3, top_p=0.75, lib=lib)
        want = p4[token] / p4[:2].sum() if token < 2 else 0.0
        assert abs(r["p_at_draft"][0, 0] - want) < 1e-9, token


def check_min_p_closed_form(lib):
    """min_p = 0.5 on p = (.5, .3, .2) keeps p >= .25: {0, 1}; at temperature 2 the
    threshold is on p = softmax(x / 2)."""
    base = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32)
    for T in (1.0, 2.0):
        p = lib_softmax(base, T)
        kept = p >= 0.5 * p.max()
        for token in range(3):
            t, d, x, u = _one_row_case(base, base, token)
            r = oracle.stochastic(t, d, x, u, T, min_p=0.5, lib=lib)
            want = p[token] / p[kept].sum() if kept[token] else 0.0
            assert abs(r["p_at_draft"][0, 0] - want) < 1e-9, (T, token)


def check_filtered_output_distribution(lib, trials: int = 400_000):
    """Chi-squared: with both sides filtered (top-k 5, top-p 0.9) and x ~ q', the first
    emitted token is distributed as p', the filtered target (p' from a sort of the
    library softmax)."""
    rng = np.random.default_rng(53)
    V = 8
    tl = rng.normal(0, 1.2, (2, V)).astype(np.float32)
    dl = (tl[:1] + rng.normal(0, 1.0, (1, V))).astype(np.float32)

    def filtered(logits):
        p = lib_softmax(logits)
        order = np.argsort(-logits, kind="stable")
        keep = np.zeros(V, bool)
        keep[order[:5]] = True
        p5 = np.where(keep, p, 0.0) / p[keep].sum()
        cum = np.cumsum(p5[order])
        cut = order[: int(np.searchsorted(cum, 0.9)) + 1]
        out = np.zeros(V)
        out[cut] = p[cut]
        return out / out.sum()

    pf, qf = filtered(tl[0]), filtered(dl[0])
    x = sample_from(rng, qf, trials).reshape(trials, 1)
    u = rng.random((trials, 2), dtype=np.float32)
    t = np.broadcast_to(tl, (trials, 2, V)).copy()
    d = np.broadcast_to(dl, (trials, 1, V)).copy()
    r = oracle.stochastic(t, d, x, u, 1.0, top_k=5, top_p=0.9, lib=lib)
    assert chi2_stat(np.bincount(r["out_tokens"][:, 0], minlength=V), pf) < CHI2_DF7_P001


# ---- guard band: the margins that classify a request as ambiguous --------------
#
# A request is ambiguous when a decision it actually took lies within 1e-6 of
# its boundary: test i at u_i against min(1, P/Q) (the strict test
# u < min(1, p(x)/q(x)) of "02. Speculative Decoding", section 2), the final
# draw at u*Z against the nearer edge of the chosen token's CDF interval,
# relative to Z.  The values below come from hand-built rows whose P/Q is
# known in closed form, and from searchsorted over library cumulative sums.

def _exact_rows():
    """One target row p = (1/4, 3/4, 0, 0) and draft rows q = (1, 0, 0, 0) and
    q' = (1/8, 7/8, 0, 0): P/Q = 1/4 for token 0 under q, P/Q = 6/7 for token 1
    under q', P >= Q for token 1 under q."""
    t = np.array([0.0, np.log(3.0), -np.inf, -np.inf], np.float32)
    q = np.array([0.0, -np.inf, -np.inf, -np.inf], np.float32)
    q2 = np.array([0.0, np.log(7.0), -np.inf, -np.inf], np.float32)
    p = lib_softmax(t)
    return t, q, q2, p


def check_accept_margin(lib):
    """margin[i] = |u - min(1, P/Q)| for the test actually taken: u = P/Q +- delta
    for several delta (P/Q from the library softmax of the float32 rows), u
    against 1 when P >= Q, and +inf past the stop row."""
    t, q, q2, p = _exact_rows()
    pq = lib_softmax(q)
    pq2 = lib_softmax(q2)
    cases = [(q, 0, p[0] / pq[0]), (q2, 1, p[1] / pq2[1]), (q, 1, 1.0)]  # (draft, token, threshold)
    for draft, token, thr in cases:
        for delta in (0.25e-1, -0.125, 3e-6, -2e-6, 7e-7, -4e-7):
            u0 = np.float32(min(max(thr + delta, 0.0), 0.99999994))
            tt = np.stack([t, t])[None]  # k = 1: row 0 tested, row 1 bonus
            r = oracle.stochastic(tt, draft[None, None], np.array([[token]], np.int32),
                                  np.array([[u0, 0.5]], np.float32), 1.0, lib=lib)
            want = abs(float(u0) - min(1.0, thr))
            assert abs(r["margins"][0, 0] - want) < 1e-12, (token, delta, r["margins"][0, 0], want)
    # past the stop row: +inf (k = 2, test 0 rejects with u near 1)
    tt = np.stack([t, t, t])[None]
    dd = np.stack([q, q])[None]
    r = oracle.stochastic(tt, dd, np.array([[0, 0]], np.int32),
                          np.array([[0.9, 0.1, 0.5]], np.float32), 1.0, lib=lib)
    assert r["num_accepted"][0] == 0 and np.isinf(r["margins"][0, 1])


def check_final_margin(lib):
    """margin[k] = distance from u*Z to the nearest CDF edge divided by Z, from
    searchsorted over library cumulative sums: residual draws (Z < 1, so the
    division matters) on rows with zero weights, and bonus draws."""
    rng = np.random.default_rng(81)
    B, V = 400, 12
    tl = rng.normal(0, 1.0, (B, 2, V)).astype(np.float32)
    dl = rng.normal(0, 1.0, (B, 1, V)).astype(np.float32)
    tl[:, :, 0] = -np.inf  # token 0 never has weight
    tl[rng.random((B, 2, V)) < 0.2] = -np.inf
    tl[:, :, 1] = 0.5      # every row keeps a finite logit
    x = rng.integers(0, V, (B, 1)).astype(np.int32)
    u = rng.random((B, 2), dtype=np.float32)
    r = oracle.stochastic(tl, dl, x, u, 1.0, lib=lib)
    p = lib_softmax(tl)
    q = lib_softmax(dl)
    n_res = 0
    for b in range(B):
        s = int(r["num_accepted"][b])
        if s == 0:
            w = np.maximum(p[b, 0] - q[b, 0], 0.0)
            if not w.sum() > 0:
                continue
            n_res += 1
        else:
            w = p[b, 1]
        j, dist = lib_inverse_cdf(w, float(u[b, 1]))
        assert abs(r["margins"][b, 1] - dist) < 1e-9 * max(1.0, dist), (b, s)
        if dist > 1e-9:
            assert r["out_tokens"][b, s] == j, b
    assert n_res > 50


def check_top_p_margin(lib):
    """filter_margins of a top-p row: the distance of the target top_p * mass1
    from the nearer cumulative edge of the group it falls in, divided by mass1
    (the mass of the top-k survivors), from a sort of the library softmax."""
    base = np.log(np.array([0.35, 0.25, 0.2, 0.12, 0.08])).astype(np.float32)
    p = lib_softmax(base)
    for top_k, top_p in ((0, 0.5), (0, 0.83), (3, 0.7), (4, 0.95), (3, 0.4)):
        keep = np.arange(5) < (top_k if top_k else 5)
        mass1 = p[keep].sum()
        cum = np.concatenate([[0.0], np.cumsum(p[keep])])
        target = float(np.float32(top_p)) * mass1
        g = int(np.searchsorted(cum, target, side="left"))  # first edge >= target
        want = min(target - cum[g - 1], cum[g] - target) / mass1
        r = oracle.stochastic(base[None, None], None, np.zeros((1, 0), np.int32),
                              np.array([[0.3]], np.float32), 1.0, top_k=top_k,
                              top_p=float(np.float32(top_p)), lib=lib)
        assert abs(r["filter_margins"][0] - want) < 1e-12, (top_k, top_p,
                                                            r["filter_margins"][0], want)


def check_min_p_margin(lib):
    """filter_margins of a min-p row: the smallest |x - (max x + T ln(min_p))| over
    the row's logits (absolute, logit units), at two temperatures."""
    rng = np.random.default_rng(83)
    for T, min_p in ((1.0, 0.5), (0.7, 0.05)):
        x = rng.normal(0, 1.0, 9).astype(np.float32)
        x[0] = np.float32(2.0)
        tmin = 2.0 + T * np.log(np.float32(min_p), dtype=np.float64)
        x[4] = np.float32(tmin + 3e-3)  # one logit a known distance above the threshold
        want = float(np.min(np.abs(x.astype(np.float64) - tmin)))
        assert want <= 3.1e-3
        r = oracle.stochastic(x[None, None], None, np.zeros((1, 0), np.int32),
                              np.array([[0.3]], np.float32), T, min_p=float(np.float32(min_p)),
                              lib=lib)
        assert abs(r["filter_margins"][0] - want) < 1e-12, (T, r["filter_margins"][0], want)


def check_ambiguous_requests(lib, fn=None):
    """The classifier: a request is ambiguous iff its smallest decision margin is
    strictly below the band (or, for filtered calls, its filter margin below the
    filter band); +inf margins (decisions not taken) never count."""
    fn = fn or oracle.ambiguous_requests
    inf = np.inf
    margins = np.array([[inf, 5e-7, inf],   # one decision inside the band
                        [2e-6, 3e-6, inf],  # all outside
                        [1e-6, inf, 4e-6],  # exactly on the band: outside (strict)
                        [inf, inf, inf],    # no decision taken
                        [0.0, 0.5, 0.5]])   # a decision on its boundary
    np.testing.assert_array_equal(fn(margins, 1e-6), [True, False, False, False, True])
    fm = np.array([inf, 1e-10, 1e-9, 2.0, inf])
    np.testing.assert_array_equal(fn(margins, 1e-6, fm, 1e-9), [True, True, False, False, True])
    del lib


def check_tree_sibling_margins(lib):
    """Stochastic tree margins: the first child's test against min(1, p/q), the
    second sibling's against min(1, r/q) with r the normalised residual (library
    softmax), the final draw's from searchsorted over the second residual."""
    V = 4
    tl = np.log(np.array([[0.4, 0.1, 0.3, 0.2]] + [[0.25] * V] * 2)).astype(np.float32)
    dl = np.log(np.array([[0.1, 0.5, 0.25, 0.15]] + [[0.25] * V] * 2)).astype(np.float32)
    p = lib_softmax(tl[0])
    q = lib_softmax(dl[0])
    res = np.maximum(p - q, 0.0)
    res /= res.sum()
    res2 = np.maximum(res - q, 0.0)
    thr1, thr2 = p[1] / q[1], res[2] / q[2]
    paths = np.array([[[0, 1], [0, 2]]], np.int32)
    tok = np.array([[0, 1, 2]], np.int32)
    u = np.array([[0.999, min(thr2 * 1.01, 0.999), 0.6]], np.float32)
    r = oracle.tree_stochastic(tl[None], dl[None], tok, paths, u, 1.0, lib=lib)
    assert r["num_accepted"][0] == 0
    assert abs(r["margins"][0, 0] - abs(float(u[0, 0]) - thr1)) < 1e-12
    assert abs(r["margins"][0, 1] - abs(float(u[0, 1]) - thr2)) < 1e-12
    _, dist = lib_inverse_cdf(res2, float(u[0, 2]))
    assert abs(r["margins"][0, 2] - dist) < 1e-12


# ---- stochastic tree ----------------------------------------------------------

def _chain_paths(B, k, P=3):
    paths = np.full((B, P, k + 1), -1, np.int32)
    paths[:, 1, :] = np.arange(k + 1)
    return paths


def check_tree_stochastic_chain_is_linear(lib):
    """A single-chain tree is the linear stochastic verification on the same rows
    (same tokens, accept counts and margins), f32 and bf16."""
    rng = np.random.default_rng(61)
    for dtype, V, k, T in (("f32", 40, 4, 1.0), ("bf16", 300, 3, 0.8), ("f32", 7, 6, 1.3)):
        B = 64
        t32 = rng.normal(0, 2, (B, k + 1, V)).astype(np.float32)
        d32 = (t32 + rng.normal(0, 1, (B, k + 1, V))).astype(np.float32)
        t = to_bf16_bits(t32) if dtype == "bf16" else t32
        d = to_bf16_bits(d32) if dtype == "bf16" else d32
        qf = lib_softmax(bf16_bits_to_f64(d) if dtype == "bf16" else d, T)
        x = np.stack([[sample_from(rng, qf[b, i], 1)[0] for i in range(k)] for b in range(B)])
        x = x.astype(np.int32)
        x[rng.random((B, k)) < 0.05] = V  # a few ids outside the vocabulary
        u = rng.random((B, k + 1), dtype=np.float32)
        tok = np.concatenate([np.zeros((B, 1), np.int32), x], axis=1)
        r = oracle.tree_stochastic(t, d, tok, _chain_paths(B, k), u, T, lib=lib)
        g = oracle.stochastic(t, d[:, :k], x, u, T, lib=lib)
        np.testing.assert_array_equal(r["num_accepted"], g["num_accepted"])
        np.testing.assert_array_equal(r["out_tokens"], g["out_tokens"])
        np.testing.assert_array_equal(r["margins"], g["margins"])
        for b in range(B):
            s = int(r["num_accepted"][b])
            assert r["accepted_nodes"][b, :s].tolist() == list(range(1, s + 1))
            assert np.all(r["accepted_nodes"][b, s:] == -1)


def check_tree_stochastic_sibling_residual(lib):
    """Root with two children: the first child is rejected (u above P/Q), the
    second is tested against normalise(max(0, p - q)) (closed form from the library
    softmax), on both sides of its threshold."""
    V = 4
    tl = np.log(np.array([[0.4, 0.1, 0.3, 0.2]] + [[0.25] * V] * 2)).astype(np.float32)
    dl = np.log(np.array([[0.1, 0.5, 0.25, 0.15]] + [[0.25] * V] * 2)).astype(np.float32)
    p = lib_softmax(tl[0])
    q = lib_softmax(dl[0])
    x1, x2 = 1, 2
    assert p[x1] < q[x1]
    res = np.maximum(p - q, 0.0)
    res /= res.sum()
    assert res[x2] < q[x2] and res[x2] > 0
    thr = res[x2] / q[x2]
    paths = np.array([[[0, 1], [0, 2]]], np.int32)
    tok = np.array([[0, x1, x2]], np.int32)
    for u2, want in ((thr * 0.999, 1), (min(thr * 1.001, 0.999), 0)):
        u = np.array([[0.999, u2, 0.25]], np.float32)
        r = oracle.tree_stochastic(tl[None], dl[None], tok, paths, u, 1.0, lib=lib)
        if want:
            assert r["num_accepted"][0] == 1 and r["accepted_nodes"][0, 0] == 2
            assert r["out_tokens"][0, 0] == x2
        else:
            # both rejected: the final draw is from the second residual
            assert r["num_accepted"][0] == 0
            res2 = np.maximum(res - q, 0.0)
            j, _ = lib_inverse_cdf(res2, 0.25)
            assert r["out_tokens"][0, 0] == j


def check_tree_stochastic_output_distribution(lib, trials: int = 300_000):
    """Chi-squared: three children drawn independently from q at the root; the
    first emitted token (an accepted child's, or the final draw) is distributed as
    p (the property the rule is built for)."""
    rng = np.random.default_rng(67)
    V, m = 8, 3
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
    r = oracle.tree_stochastic(t, d, tok, paths, u, 1.0, lib=lib)
    assert chi2_stat(np.bincount(r["out_tokens"][:, 0], minlength=V), p) < CHI2_DF7_P001


def check_tree_stochastic_identical_draft(lib):
    """q = p at every node: the first child of each node is always accepted and the
    walk follows first children to a leaf."""
    rng = np.random.default_rng(71)
    B, V = 32, 30
    N = 6  # 0 -> {1, 2}, 1 -> {3, 4}, 3 -> {5}, 2 -> {6}
    parent = [-1, 0, 0, 1, 1, 3, 2]
    t = rng.normal(0, 2, (B, N + 1, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, N + 1)).astype(np.int32)
    paths = np.full((B, 3, 4), -1, np.int32)
    paths[:, 0] = [0, 1, 3, 5]
    paths[:, 1] = [0, 1, 4, -1]
    paths[:, 2] = [0, 2, 6, -1]
    u = rng.random((B, N + 1), dtype=np.float32)
    r = oracle.tree_stochastic(t, t.copy(), tok, paths, u, 1.0, lib=lib)
    assert np.all(r["num_accepted"] == 3)
    assert np.all(r["accepted_nodes"][:, :3] == [1, 3, 5])
    np.testing.assert_array_equal(r["out_tokens"][:, :3], tok[:, [1, 3, 5]])
    for b in range(B):  # the final draw is from the leaf's target row
        j, _ = lib_inverse_cdf(lib_softmax(t[b, 5]), float(u[b, N]))
        assert r["out_tokens"][b, 3] == j
    assert parent[5] == 3


def check_gather_rows_example(lib):
    """Accepted-row gather on a hand-built case: request 0 keeps nodes 3 and 1 in
    that order, request 1 none, request 2 node 2; other rows stay untouched."""
    src = np.arange(3 * 4 * 2, dtype=np.int32).reshape(3, 4, 2)  # row (b, n) = [8b+2n, 8b+2n+1]
    nodes = np.array([[3, 1, -1], [-1, -1, -1], [2, -1, -1]], np.int32)
    acc = np.array([2, 0, 1], np.int32)
    dst = np.full((3, 3, 2), -7, np.int32)
    out = oracle.gather_rows(src, nodes, acc, dst)
    want = np.full((3, 3, 2), -7, np.int32)
    want[0, 0] = [6, 7]
    want[0, 1] = [2, 3]
    want[2, 0] = [20, 21]
    np.testing.assert_array_equal(out, want)


ALL_CHECKS = [
    check_softmax_vs_library,
    check_identical_draft_accepts_all,
    check_disjoint_support_rejects_first,
    check_one_hot_draft_closed_form,
    check_strict_threshold,
    check_acceptance_frequency,
    check_emitted_tokens_distributed_as_p,
    check_inverse_cdf_zero_weights,
    check_out_of_range_draft_rejected,
    check_fgxy_worked_example,
    check_greedy_argmax_chain,
    check_tree_bruteforce,
    check_chain_tree_equals_greedy,
    check_tree_unused_rows,
    check_ragged_is_each_request_alone,
    check_ragged_zero_length_samples_row_zero,
    check_greedy_ragged,
    check_philox_matches_numpy,
    check_philox_uniform_layout,
    check_filter_off_is_plain,
    check_top_k_closed_form,
    check_top_p_closed_form,
    check_min_p_closed_form,
    check_filtered_output_distribution,
    check_tree_stochastic_chain_is_linear,
    check_tree_stochastic_sibling_residual,
    check_tree_stochastic_output_distribution,
    check_tree_stochastic_identical_draft,
    check_gather_rows_example,
    check_accept_margin,
    check_final_margin,
    check_top_p_margin,
    check_min_p_margin,
    check_ambiguous_requests,
    check_tree_sibling_margins,
]
