"""CPU oracle for batched draft-token verification: ctypes binding.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The oracle itself is ``spec_verify_oracle.c`` (plain C, fp64, scalar
loops); this module only compiles it with gcc and marshals NumPy arrays.

Logits are passed as NumPy ``float32`` arrays or as ``uint16`` arrays holding
raw bf16 bit patterns (the oracle widens bf16 to double itself).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_verify_oracle.c")
_LIB = os.path.join(_HERE, "libspec_verify_oracle.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

SOURCE = _SRC


def compile_source(src: str, out: str) -> str:
    """gcc a C source of the oracle into a shared library at ``out``."""
    tmp = out + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", src, "-o", tmp,
         "-lm"],
        check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libspec_verify_oracle.so``."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def _open(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_verify_stochastic.argtypes = [P, P, i, P, P, ctypes.c_double, i, i, i,
                                             P, P, P, P, P]
    lib.oracle_verify_stochastic.restype = i
    lib.oracle_verify_greedy.argtypes = [P, i, P, i, i, i, P, P, P]
    lib.oracle_verify_greedy.restype = i
    lib.oracle_verify_stochastic_ragged.argtypes = [P, P, i, P, P, P, ctypes.c_double, i, i, i,
                                                    P, P, P, P, P]
    lib.oracle_verify_stochastic_ragged.restype = i
    lib.oracle_verify_greedy_ragged.argtypes = [P, i, P, P, i, i, i, P, P, P]
    lib.oracle_verify_greedy_ragged.restype = i
    lib.oracle_verify_stochastic_filtered.argtypes = [P, P, i, P, P, ctypes.c_double, i,
                                                      ctypes.c_double, ctypes.c_double, i, i, i,
                                                      P, P, P, P, P, P]
    lib.oracle_verify_stochastic_filtered.restype = i
    lib.oracle_philox4x64_10.argtypes = [P, P, P]
    lib.oracle_philox4x64_10.restype = None
    lib.oracle_philox_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, i, i, P]
    lib.oracle_philox_uniforms.restype = None
    lib.oracle_verify_tree.argtypes = [P, i, P, P, i, i, i, i, i, P, P, P, P]
    lib.oracle_verify_tree.restype = i
    lib.oracle_verify_tree_stochastic.argtypes = [P, P, i, P, P, P, ctypes.c_double, i, i, i, i,
                                                  i, P, P, P, P]
    lib.oracle_verify_tree_stochastic.restype = i
    return lib


_default = None


def _load():
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _default = _open(_LIB)
    return _default


def _logits(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, DTYPE_F32
    if a.dtype == np.uint16:
        return a, DTYPE_BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def open_library(path: str):
    """Load another build of the oracle (used to check that planted mistakes are caught)."""
    return _open(path)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def stochastic(target_logits, draft_logits, draft_tokens, uniforms, temperature, *,
               draft_lens=None, top_k=0, top_p=1.0, min_p=0.0, lib=None):
    """Oracle stochastic verify.

    Returns ``dict(out_tokens[B,k+1] int32, num_accepted[B] int32,
    p_at_draft[B,k] f64, q_at_draft[B,k] f64, margins[B,k+1] f64)``.
    With ``draft_lens`` ([B] ints), request b uses only its first
    ``draft_lens[b]`` drafts (clamped to [0, k]).  With ``top_k``, ``top_p`` or
    ``min_p`` set, every row is filtered first and the result also holds
    ``filter_margins[B]``.
    """
    filtered = top_k != 0 or top_p != 1.0 or min_p != 0.0
    t, dt = _logits(target_logits)
    B, k1, V = t.shape
    k = k1 - 1
    if k > 0:
        d, dd = _logits(draft_logits)
        assert dd == dt and d.shape == (B, k, V)
    else:
        d = np.zeros((B, 0, V), dtype=t.dtype)
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, k)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, k + 1)
    out = np.empty((B, k + 1), np.int32)
    acc = np.empty((B,), np.int32)
    pp = np.empty((B, k), np.float64)
    qq = np.empty((B, k), np.float64)
    mg = np.empty((B, k + 1), np.float64)
    fm = np.full((B,), np.inf, np.float64)
    if filtered:
        assert draft_lens is None, "filtering with ragged lengths is not modelled"
        rc = (lib or _load()).oracle_verify_stochastic_filtered(
            _ptr(t), _ptr(d), dt, _ptr(x), _ptr(u), float(temperature), int(top_k),
            float(top_p), float(min_p), B, k, V, _ptr(out), _ptr(acc), _ptr(pp), _ptr(qq),
            _ptr(mg), _ptr(fm))
    elif draft_lens is None:
        rc = (lib or _load()).oracle_verify_stochastic(
            _ptr(t), _ptr(d), dt, _ptr(x), _ptr(u), float(temperature), B, k, V, _ptr(out),
            _ptr(acc), _ptr(pp), _ptr(qq), _ptr(mg))
    else:
        ln = np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
        rc = (lib or _load()).oracle_verify_stochastic_ragged(
            _ptr(t), _ptr(d), dt, _ptr(x), _ptr(ln), _ptr(u), float(temperature), B, k, V,
            _ptr(out), _ptr(acc), _ptr(pp), _ptr(qq), _ptr(mg))
    if rc != 0:
        raise ValueError(f"oracle_verify_stochastic failed with code {rc}")
    return dict(out_tokens=out, num_accepted=acc, p_at_draft=pp, q_at_draft=qq, margins=mg,
                filter_margins=fm)


def greedy(target_logits, draft_tokens, *, draft_lens=None, lib=None):
    """Oracle greedy verify: ``dict(out_tokens, num_accepted, argmax[B,k+1])``; with
    ``draft_lens``, request b uses only its first ``draft_lens[b]`` drafts."""
    t, dt = _logits(target_logits)
    B, k1, V = t.shape
    k = k1 - 1
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, k)
    out = np.empty((B, k + 1), np.int32)
    acc = np.empty((B,), np.int32)
    am = np.empty((B, k + 1), np.int32)
    if draft_lens is None:
        rc = (lib or _load()).oracle_verify_greedy(
            _ptr(t), dt, _ptr(x), B, k, V, _ptr(out), _ptr(acc), _ptr(am))
    else:
        ln = np.ascontiguousarray(draft_lens, dtype=np.int32).reshape(B)
        rc = (lib or _load()).oracle_verify_greedy_ragged(
            _ptr(t), dt, _ptr(x), _ptr(ln), B, k, V, _ptr(out), _ptr(acc), _ptr(am))
    if rc != 0:
        raise ValueError(f"oracle_verify_greedy failed with code {rc}")
    return dict(out_tokens=out, num_accepted=acc, argmax=am)


def philox4x64_10(counter, key, *, lib=None) -> np.ndarray:
    """One Philox4x64-10 block: four uint64 words for a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(counter, dtype=np.uint64).reshape(4)
    k = np.ascontiguousarray(key, dtype=np.uint64).reshape(2)
    out = np.empty(4, np.uint64)
    (lib or _load()).oracle_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox_uniforms(seed: int, offset: int, B: int, n: int, *, lib=None) -> np.ndarray:
    """uniforms[B, n] float32 of request b, draw i: counter (offset, b, i // 4, 0),
    key (seed, 0), word i % 4, (word >> 40) * 2^-24."""
    out = np.empty((B, n), np.float32)
    (lib or _load()).oracle_philox_uniforms(ctypes.c_uint64(seed), ctypes.c_uint64(offset), B,
                                            n, _ptr(out))
    return out


def tree(target_logits, node_tokens, paths, *, lib=None):
    """Oracle tree verify: ``dict(out_tokens[B,L], num_accepted, best_path, accepted_nodes)``."""
    t, dt = _logits(target_logits)
    B, N1, V = t.shape
    N = N1 - 1
    nt = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N1)
    pa = np.ascontiguousarray(paths, dtype=np.int32)
    assert pa.ndim == 3 and pa.shape[0] == B
    P, L = pa.shape[1], pa.shape[2]
    out = np.empty((B, L), np.int32)
    acc = np.empty((B,), np.int32)
    best = np.empty((B,), np.int32)
    nodes = np.empty((B, L), np.int32)
    rc = (lib or _load()).oracle_verify_tree(
        _ptr(t), dt, _ptr(nt), _ptr(pa), B, N, P, L, V, _ptr(out), _ptr(acc), _ptr(best),
        _ptr(nodes))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree failed with code {rc}")
    return dict(out_tokens=out, num_accepted=acc, best_path=best, accepted_nodes=nodes)


def tree_stochastic(target_logits, draft_logits, node_tokens, paths, uniforms, temperature, *,
                    lib=None):
    """Oracle stochastic tree verify (multi-candidate speculative sampling over
    each accepted node's children): ``dict(out_tokens[B,L], num_accepted[B],
    accepted_nodes[B,L], margins[B,N+1])``; ``uniforms[b, c-1]`` drives node c's
    test, ``uniforms[b, N]`` the final draw."""
    t, dt = _logits(target_logits)
    B, N1, V = t.shape
    N = N1 - 1
    d, dd = _logits(draft_logits)
    assert dd == dt and d.shape == t.shape
    nt = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N1)
    pa = np.ascontiguousarray(paths, dtype=np.int32)
    assert pa.ndim == 3 and pa.shape[0] == B
    P, L = pa.shape[1], pa.shape[2]
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, N1)
    out = np.empty((B, L), np.int32)
    acc = np.empty((B,), np.int32)
    nodes = np.empty((B, L), np.int32)
    mg = np.empty((B, N1), np.float64)
    rc = (lib or _load()).oracle_verify_tree_stochastic(
        _ptr(t), _ptr(d), dt, _ptr(nt), _ptr(pa), _ptr(u), float(temperature), B, N, P, L, V,
        _ptr(out), _ptr(acc), _ptr(nodes), _ptr(mg))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_stochastic failed with code {rc}")
    return dict(out_tokens=out, num_accepted=acc, accepted_nodes=nodes, margins=mg)


def gather_rows(src, accepted_nodes, num_accepted, dst):
    """Oracle accepted-row gather: ``dst[b, j] = src[b, accepted_nodes[b, j]]`` for
    ``j < num_accepted[b]``; other rows of ``dst`` are left as they are."""
    out = np.array(dst, copy=True)
    for b in range(src.shape[0]):
        for j in range(int(num_accepted[b])):
            out[b, j] = src[b, accepted_nodes[b, j]]
    return out


def ambiguous_requests(margins: np.ndarray, band: float = 1e-6, filter_margins=None,
                       filter_band: float = 1e-9) -> np.ndarray:
    """Boolean [B]: some decision actually taken lies within ``band`` of its boundary,
    or (filtered calls) a filter threshold lies within ``filter_band`` of flipping.

    The decisions taken by request b are tests 0..min(s, k-1) and the final
    sample; untaken tests carry +inf margins, so the row minimum suffices.
    """
    amb = np.min(margins, axis=1) < band
    if filter_margins is not None:
        amb |= np.asarray(filter_margins) < filter_band
    return amb
