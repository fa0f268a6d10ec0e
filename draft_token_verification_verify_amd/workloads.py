"""Seeded synthetic inputs for draft-token verification.

This module only draws inputs.  It holds none of the verification arithmetic
(no softmax, no acceptance test, no residual or inverse-CDF sampling); both the
HIP path's tests and the oracle's tests take their inputs from here.

Every array is NumPy.  Randomness is NumPy's PCG64 (``default_rng(seed)``).
bf16 tensors are made by a round-to-nearest-even cast of float32 (PyTorch's
``.to(torch.bfloat16)``) and are carried as ``uint16`` bit patterns.  Draft
tokens of stochastic workloads are draws from softmax(draft / T), taken with the
Gumbel-max trick (argmax of logits / T plus iid standard Gumbel noise), which is
an exact sampler for that distribution.

Workloads (sizes as in the verification step of a speculative decoder):
  * ``c1``: stochastic, B=1, k=3, V=1000, fp32; target ~ N(0, sd 2);
    draft = target + N(0, sd 0.5); T = 1.
  * ``c2``: greedy and stochastic, B=8, k=4, V=32000, bf16; target ~ N(0, sd 3);
    draft = target + N(0, sd 1); target rows with a tied bf16 maximum are
    redrawn; greedy drafts are argmax(draft), stochastic drafts are sampled;
    T = 1.
  * ``c3``: stochastic, B=64, k=3, V=128256, bf16, T = 0.8; rank-Zipf target
    -1.1 ln(pi_j) + N(0, sd 0.3) with one random permutation pi of 1..V per seed
    shared by all rows; draft = target + N(0, sd 1).
  * ``c4``: stochastic, B=256, k=5, V=151936, fp32, T = 1; as c3 but a fresh
    permutation per target row; draft = 0.7 target + N(0, sd 1.5).
  * ``c5``: tree greedy, B=32, 60 draft nodes of depth exactly 6 with at most 10
    children per node, V=128256, bf16; target ~ N(0, sd 3) over 61 rows;
    paths[32, 60, 7] one row per leaf, root first, -1 padded; a node's token is
    the argmax of its parent's row with probability 0.6, else uniform in [0, V).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "StochasticCase", "GreedyCase", "TreeCase",
    "gaussian_stochastic", "zipf_stochastic", "gaussian_greedy", "random_tree_case",
    "c1", "c2_greedy", "c2_stochastic", "c3", "c4", "c5", "stochastic_tree_case",
    "StochasticTreeCase",
    "bf16_bits", "bits_to_float", "to_device",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even) and return the uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_device(a: np.ndarray, dtype: str | None = None, device="cuda"):
    """Copy a NumPy array to a torch device tensor; ``dtype="bf16"`` reinterprets
    uint16 bit patterns as torch.bfloat16."""
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class StochasticCase:
    name: str
    B: int
    k: int
    V: int
    dtype: str                 # "f32" or "bf16"
    temperature: float
    target: np.ndarray         # [B, k+1, V] float32, or uint16 bf16 bits
    draft: np.ndarray          # [B, k, V]
    draft_tokens: np.ndarray   # [B, k] int32
    uniforms: np.ndarray       # [B, k+1] float32 in [0, 1)
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.B * (self.k + 1)

    @property
    def logits_bytes(self) -> int:
        return self.target.nbytes + self.draft.nbytes


@dataclass
class GreedyCase:
    name: str
    B: int
    k: int
    V: int
    dtype: str
    target: np.ndarray         # [B, k+1, V]
    draft_tokens: np.ndarray   # [B, k] int32
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.B * (self.k + 1)

    @property
    def logits_bytes(self) -> int:
        return self.target.nbytes


@dataclass
class TreeCase:
    name: str
    B: int
    N: int
    P: int
    L: int
    V: int
    dtype: str
    target: np.ndarray         # [B, N+1, V]
    node_tokens: np.ndarray    # [B, N+1] int32
    paths: np.ndarray          # [B, P, L] int32, -1 padded
    parents: np.ndarray        # [B, N+1] int32 (-1 for the root); generator bookkeeping
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.B * (self.N + 1)

    @property
    def logits_bytes(self) -> int:
        return self.target.nbytes


def _f32(x: float) -> float:
    """The float32 value nearest x, as a Python float: the library takes the
    temperature as float32, so every consumer is given exactly that value."""
    return float(np.float32(x))


def _finish(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x32)
    raise ValueError(dtype)


def _as_float(x: np.ndarray, dtype: str) -> np.ndarray:
    return bits_to_float(x) if dtype == "bf16" else x


def _sample_drafts(rng, draft: np.ndarray, dtype: str, temperature: float) -> np.ndarray:
    """One draw per draft row from softmax(draft / T), by Gumbel-max."""
    B, k, V = draft.shape
    out = np.empty((B, k), np.int32)
    flat = draft.reshape(B * k, V)
    rows_per_chunk = max(1, (1 << 22) // max(V, 1))
    for r0 in range(0, B * k, rows_per_chunk):
        r1 = min(B * k, r0 + rows_per_chunk)
        z = _as_float(flat[r0:r1], dtype).astype(np.float64) / temperature
        g = rng.gumbel(size=z.shape)
        out.reshape(-1)[r0:r1] = np.argmax(z + g, axis=1).astype(np.int32)
    return out


def _uniforms(rng, B: int, k: int) -> np.ndarray:
    return rng.random((B, k + 1), dtype=np.float32)


def _redraw_tied_rows(rng, target32: np.ndarray, sd: float) -> np.ndarray:
    """Redraw (in place) target rows whose bf16 maximum occurs more than once."""
    flat = target32.reshape(-1, target32.shape[-1])
    for _ in range(1000):
        vals = bits_to_float(bf16_bits(flat))
        mx = vals.max(axis=1, keepdims=True)
        tied = np.nonzero((vals == mx).sum(axis=1) > 1)[0]
        if tied.size == 0:
            return target32
        flat[tied] = rng.normal(0.0, sd, size=(tied.size, flat.shape[1])).astype(np.float32)
    raise RuntimeError("could not draw rows with a unique maximum")


def gaussian_stochastic(seed: int, B: int, k: int, V: int, dtype: str, *,
                        target_sd: float, draft_noise_sd: float, temperature: float = 1.0,
                        unique_max: bool = False, name: str = "gaussian") -> StochasticCase:
    """target ~ N(0, target_sd) iid; draft = target[:, :k] + N(0, draft_noise_sd)."""
    rng = np.random.default_rng(seed)
    t32 = rng.normal(0.0, target_sd, size=(B, k + 1, V)).astype(np.float32)
    if unique_max:
        _redraw_tied_rows(rng, t32, target_sd)
    d32 = (t32[:, :k, :] + rng.normal(0.0, draft_noise_sd, size=(B, k, V))).astype(np.float32)
    target = _finish(t32, dtype)
    draft = _finish(d32, dtype)
    drafts = _sample_drafts(rng, draft, dtype, temperature)
    return StochasticCase(name, B, k, V, dtype, _f32(temperature), target, draft, drafts,
                          _uniforms(rng, B, k), dict(seed=seed))


def zipf_stochastic(seed: int, B: int, k: int, V: int, dtype: str, *,
                    per_row_permutation: bool, draft_scale: float, draft_noise_sd: float,
                    temperature: float, target_noise_sd: float = 0.3,
                    name: str = "zipf") -> StochasticCase:
    """Rank-Zipf logits: target[.., j] = -1.1 ln(pi_j) + N(0, target_noise_sd).

    pi is a random permutation of 1..V, one per seed (shared by every row) or one
    per target row; draft = draft_scale * target[:, :k] + N(0, draft_noise_sd).
    """
    rng = np.random.default_rng(seed)
    log_rank = np.log(np.arange(1, V + 1, dtype=np.float64)).astype(np.float32)
    rows = B * (k + 1)
    if per_row_permutation:
        ranks = rng.permuted(np.broadcast_to(log_rank, (rows, V)), axis=1)
    else:
        ranks = np.broadcast_to(rng.permutation(log_rank), (rows, V))
    t32 = (-1.1 * ranks).astype(np.float32).reshape(B, k + 1, V)
    t32 += rng.standard_normal(size=t32.shape, dtype=np.float32) * np.float32(target_noise_sd)
    d32 = t32[:, :k, :] * np.float32(draft_scale)
    d32 += rng.standard_normal(size=d32.shape, dtype=np.float32) * np.float32(draft_noise_sd)
    target = _finish(t32, dtype)
    del t32
    draft = _finish(d32, dtype)
    del d32
    drafts = _sample_drafts(rng, draft, dtype, temperature)
    return StochasticCase(name, B, k, V, dtype, _f32(temperature), target, draft, drafts,
                          _uniforms(rng, B, k), dict(seed=seed))


def gaussian_greedy(seed: int, B: int, k: int, V: int, dtype: str, *, target_sd: float,
                    draft_noise_sd: float, unique_max: bool = True,
                    name: str = "gaussian-greedy") -> GreedyCase:
    """target ~ N(0, target_sd); drafts = argmax(target[:, :k] + N(0, draft_noise_sd))."""
    rng = np.random.default_rng(seed)
    t32 = rng.normal(0.0, target_sd, size=(B, k + 1, V)).astype(np.float32)
    if unique_max:
        _redraw_tied_rows(rng, t32, target_sd)
    d32 = (t32[:, :k, :] + rng.normal(0.0, draft_noise_sd, size=(B, k, V))).astype(np.float32)
    target = _finish(t32, dtype)
    draft = _as_float(_finish(d32, dtype), dtype)
    drafts = np.argmax(draft, axis=2).astype(np.int32).reshape(B, k)
    return GreedyCase(name, B, k, V, dtype, target, drafts, dict(seed=seed))


def _random_tree(rng, N: int, depth: int, max_children: int):
    """Parents of a random tree with N+1 nodes (node 0 the root), BFS numbered.

    A root-to-depth chain is laid first so the tree has exactly ``depth``
    levels; each further node hangs off a uniformly chosen node of depth <
    ``depth`` that has fewer than ``max_children`` children.
    """
    parent = [-1]
    level = [0]
    nchild = [0]
    for d in range(1, depth + 1):
        parent.append(len(parent) - 1)
        level.append(d)
        nchild.append(0)
        nchild[parent[-1]] += 1
    while len(parent) < N + 1:
        cand = [n for n in range(len(parent)) if level[n] < depth and nchild[n] < max_children]
        p = cand[int(rng.integers(0, len(cand)))]
        parent.append(p)
        level.append(level[p] + 1)
        nchild.append(0)
        nchild[p] += 1
    children = [[] for _ in parent]
    for n in range(1, len(parent)):
        children[parent[n]].append(n)
    order = [0]
    for n in order:
        order.extend(children[n])
    new_id = {old: new for new, old in enumerate(order)}
    bfs_parent = np.full(N + 1, -1, np.int32)
    for old in range(1, N + 1):
        bfs_parent[new_id[old]] = new_id[parent[old]]
    return bfs_parent


def _paths_of(parent: np.ndarray, P: int, L: int) -> np.ndarray:
    """One row per leaf (ascending node index), root first, -1 padded."""
    n_nodes = parent.shape[0]
    has_child = np.zeros(n_nodes, bool)
    has_child[parent[parent >= 0]] = True
    leaves = [n for n in range(n_nodes) if not has_child[n]]
    if len(leaves) > P:
        raise ValueError("more leaves than path rows")
    paths = np.full((P, L), -1, np.int32)
    for r, leaf in enumerate(leaves):
        chain = []
        n = leaf
        while n >= 0:
            chain.append(n)
            n = parent[n]
        chain.reverse()
        if len(chain) > L:
            raise ValueError("path longer than max_path_len")
        paths[r, :len(chain)] = chain
    return paths


def random_tree_case(seed: int, B: int, N: int, depth: int, V: int, dtype: str, *,
                     P: int | None = None, max_children: int = 10, target_sd: float = 3.0,
                     p_match: float = 0.6, name: str = "tree") -> TreeCase:
    rng = np.random.default_rng(seed)
    P = N if P is None else P
    L = depth + 1
    t32 = rng.normal(0.0, target_sd, size=(B, N + 1, V)).astype(np.float32)
    target = _finish(t32, dtype)
    del t32
    tf = _as_float(target, dtype)
    row_argmax = np.argmax(tf, axis=2).astype(np.int32)  # [B, N+1]
    parents = np.empty((B, N + 1), np.int32)
    paths = np.empty((B, P, L), np.int32)
    tokens = np.empty((B, N + 1), np.int32)
    for b in range(B):
        par = _random_tree(rng, N, depth, max_children)
        parents[b] = par
        paths[b] = _paths_of(par, P, L)
        tokens[b, 0] = int(rng.integers(0, V))
        for n in range(1, N + 1):
            if rng.random() < p_match:
                tokens[b, n] = row_argmax[b, par[n]]
            else:
                tokens[b, n] = int(rng.integers(0, V))
    return TreeCase(name, B, N, P, L, V, dtype, target, tokens, paths, parents, dict(seed=seed))


@dataclass
class StochasticTreeCase:
    name: str
    B: int
    N: int
    P: int
    L: int
    V: int
    dtype: str
    temperature: float
    target: np.ndarray         # [B, N+1, V]
    draft: np.ndarray          # [B, N+1, V]: row n, the distribution n's children come from
    node_tokens: np.ndarray    # [B, N+1] int32
    paths: np.ndarray          # [B, P, L] int32, -1 padded
    uniforms: np.ndarray       # [B, N+1] float32
    parents: np.ndarray        # [B, N+1] int32; generator bookkeeping
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.B * (self.N + 1)

    @property
    def logits_bytes(self) -> int:
        return self.target.nbytes + self.draft.nbytes


def stochastic_tree_case(seed: int, B: int, N: int, depth: int, V: int, dtype: str, *,
                         P: int | None = None, max_children: int = 10, target_sd: float = 3.0,
                         draft_noise_sd: float = 1.0, temperature: float = 1.0,
                         name: str = "stree") -> StochasticTreeCase:
    """Random trees as random_tree_case; target ~ N(0, target_sd); draft = target +
    N(0, draft_noise_sd); every node's token drawn from softmax(draft row of its
    parent / T) (Gumbel-max), independently of its siblings."""
    rng = np.random.default_rng(seed)
    P = N if P is None else P
    L = depth + 1
    t32 = rng.normal(0.0, target_sd, size=(B, N + 1, V)).astype(np.float32)
    d32 = (t32 + rng.normal(0.0, draft_noise_sd, size=(B, N + 1, V))).astype(np.float32)
    target = _finish(t32, dtype)
    draft = _finish(d32, dtype)
    del t32, d32
    dfl = _as_float(draft, dtype)
    parents = np.empty((B, N + 1), np.int32)
    paths = np.empty((B, P, L), np.int32)
    tokens = np.zeros((B, N + 1), np.int32)
    for b in range(B):
        par = _random_tree(rng, N, depth, max_children)
        parents[b] = par
        paths[b] = _paths_of(par, P, L)
        z = dfl[b, par[1:]].astype(np.float64) / temperature  # [N, V]: the parents' rows
        tokens[b, 1:] = np.argmax(z + rng.gumbel(size=z.shape), axis=1).astype(np.int32)
    u = rng.random((B, N + 1), dtype=np.float32)
    return StochasticTreeCase(name, B, N, P, L, V, dtype, _f32(temperature), target, draft,
                              tokens, paths, u, parents, dict(seed=seed))


# ---- the five named workloads -------------------------------------------------

def c1(seed: int = 0) -> StochasticCase:
    return gaussian_stochastic(seed, 1, 3, 1000, "f32", target_sd=2.0, draft_noise_sd=0.5,
                               temperature=1.0, name="c1-stochastic-B1-k3-V1000-f32")


def c2_stochastic(seed: int = 0) -> StochasticCase:
    return gaussian_stochastic(seed, 8, 4, 32000, "bf16", target_sd=3.0, draft_noise_sd=1.0,
                               temperature=1.0, unique_max=True,
                               name="c2-stochastic-B8-k4-V32000-bf16")


def c2_greedy(seed: int = 0) -> GreedyCase:
    return gaussian_greedy(seed, 8, 4, 32000, "bf16", target_sd=3.0, draft_noise_sd=1.0,
                           name="c2-greedy-B8-k4-V32000-bf16")


def c3(seed: int = 0, B: int = 64, V: int = 128256) -> StochasticCase:
    return zipf_stochastic(seed, B, 3, V, "bf16", per_row_permutation=False, draft_scale=1.0,
                           draft_noise_sd=1.0, temperature=0.8,
                           name=f"c3-stochastic-B{B}-k3-V{V}-bf16")


def c4(seed: int = 0, B: int = 256, V: int = 151936) -> StochasticCase:
    return zipf_stochastic(seed, B, 5, V, "f32", per_row_permutation=True, draft_scale=0.7,
                           draft_noise_sd=1.5, temperature=1.0,
                           name=f"c4-stochastic-B{B}-k5-V{V}-f32")


def c5(seed: int = 0, B: int = 32, V: int = 128256) -> TreeCase:
    return random_tree_case(seed, B, 60, 6, V, "bf16", P=60,
                            name=f"c5-tree-B{B}-N60-depth6-V{V}-bf16")
