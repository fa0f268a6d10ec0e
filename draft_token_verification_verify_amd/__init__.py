"""Batched draft-token verification for speculative decoding on MI355X (gfx950).

A thin binding over the C ABI in ``include/spec_verify.h``: the functions below
carry the C names, check tensor shapes, dtypes and devices, pass raw device
pointers and the current HIP stream, and return the output tensors.  Every step
of the verification runs in the library's HIP kernels; PyTorch only provides
device memory and the stream.  There is no CPU fallback: without the built
library every call raises.

    out, n = spec_verify_stochastic(target, draft, draft_tokens, uniforms, T)
    out, n = spec_verify_greedy(target, draft_tokens)
    out, n, best, nodes = spec_verify_tree(target, node_tokens, paths)
"""
from __future__ import annotations

import functools

import torch

from . import _lib
from ._lib import (BF16, F32, MODE_GREEDY, MODE_STOCHASTIC, MODE_STOCHASTIC_FILTERED, MODE_TREE,
                   MODE_TREE_STOCHASTIC, SpecVerifyError)

__all__ = [
    "spec_verify_stochastic", "spec_verify_stochastic_ragged", "spec_verify_stochastic_philox",
    "spec_verify_stochastic_filtered", "spec_verify_greedy", "spec_verify_greedy_ragged",
    "spec_verify_tree", "spec_verify_tree_stochastic", "spec_verify_tree_stochastic_split",
    "check_tree_stochastic_result", "GAVE_UP", "spec_verify_stochastic_noalloc",
    "spec_verify_gather_rows",
    "spec_verify_set_schedule",
    "spec_verify_workspace_bytes", "spec_verify_version", "Workspace", "SpecVerifyError",
    "MODE_STOCHASTIC", "MODE_GREEDY", "MODE_TREE", "MODE_STOCHASTIC_FILTERED",
    "MODE_TREE_STOCHASTIC",
]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, device: torch.device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and t.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


# The current stream's raw handle without building a Stream object (about a
# tenth of torch.cuda.current_stream's cost per call); the public call where
# torch lacks the accessor.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device, stream=None) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def spec_verify_version() -> int:
    return _lib.load().spec_verify_version()


def spec_verify_set_schedule(schedule: int) -> None:
    """Process-wide stochastic schedule: ``_lib.SCHEDULE_AUTO``,
    ``_lib.SCHEDULE_TWO_KERNELS``, ``_lib.SCHEDULE_SELF_COMPUTE`` or
    ``_lib.SCHEDULE_INTERLEAVED``."""
    _lib.check("spec_verify_set_schedule", _lib.load().spec_verify_set_schedule(int(schedule)))


@functools.lru_cache(maxsize=1024)
def spec_verify_workspace_bytes(mode: int, B: int, rows_per_request: int, V: int,
                                dtype: int) -> int:
    """Workspace bytes for a call shape (a pure function of the shape, so cached)."""
    return int(_lib.load().spec_verify_workspace_bytes(mode, B, rows_per_request, V, dtype))


class Workspace:
    """Grow-only, zero-initialised device workspaces, one buffer per (device,
    stream).

    The library leaves its counters at zero after every completed call, so one
    buffer serves every later call ordered on the same stream; calls on other
    streams get buffers of their own (two calls racing on one buffer would give
    wrong results).  Each buffer is allocated on the stream that uses it, so when
    it grows, torch's allocator does not hand the old memory to other work until
    that stream's pending calls have run.
    """

    def __init__(self):
        self._buf: dict[tuple[torch.device, int], torch.Tensor] = {}

    def get(self, nbytes: int, device: torch.device, stream=None) -> torch.Tensor:
        key = (device, _stream(device, stream))
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            s = torch.cuda.current_stream(device) if stream is None else stream
            with torch.cuda.stream(s):
                # torch.zeros clears with a fill kernel (no memset node).
                buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
            self._buf[key] = buf
        return buf


_default_workspace = Workspace()


def _workspace(ws, nbytes: int, device: torch.device, stream=None) -> torch.Tensor:
    if nbytes == 0:
        raise SpecVerifyError("spec_verify_workspace_bytes", _lib.INVALID_ARGUMENT,
                              "shape rejected by the library")
    if ws is None:
        return _default_workspace.get(nbytes, device, stream)
    if isinstance(ws, Workspace):
        return ws.get(nbytes, device, stream)
    _dev(ws, "workspace", device, torch.uint8)
    if ws.numel() < nbytes:
        raise SpecVerifyError("workspace", _lib.WORKSPACE_TOO_SMALL,
                              f"need {nbytes} bytes, got {ws.numel()}")
    return ws


def _stochastic(fn, target_logits, draft_logits, draft_tokens, draft_lens, uniforms,
                temperature, out_tokens, num_accepted, p_at_draft, q_at_draft, workspace, stream,
                seed=0, offset=0, top_k=0, top_p=1.0, min_p=0.0):
    device = target_logits.device
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, k+1, V]")
    B, k1, V = target_logits.shape
    k = k1 - 1
    _dev(target_logits, "target_logits", device)
    if k > 0:
        _dev(draft_logits, "draft_logits", device, target_logits.dtype, (B, k, V))
        _dev(draft_tokens, "draft_tokens", device, torch.int32, (B, k))
    else:
        draft_logits = draft_tokens = None
    if draft_lens is not None:
        _dev(draft_lens, "draft_lens", device, torch.int32, (B,))
    if fn != "spec_verify_stochastic_philox":
        _dev(uniforms, "uniforms", device, torch.float32, (B, k + 1))
    if out_tokens is None:
        out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=device)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=device)
    _dev(out_tokens, "out_tokens", device, torch.int32, (B, k + 1))
    _dev(num_accepted, "num_accepted", device, torch.int32, (B,))
    for name, t in (("p_at_draft", p_at_draft), ("q_at_draft", q_at_draft)):
        if t is not None:
            _dev(t, name, device, torch.float32, (B, k))
    filtered = fn == "spec_verify_stochastic_filtered"
    nbytes = spec_verify_workspace_bytes(MODE_STOCHASTIC, B, k + 1, V, dt)
    if filtered and (workspace is None or isinstance(workspace, Workspace)):
        # room for the filter candidates (a caller's own tensor may be either size)
        nbytes = spec_verify_workspace_bytes(MODE_STOCHASTIC_FILTERED, B, k + 1, V, dt)
    ws = _workspace(workspace, nbytes, device, stream)
    lib = _lib.load()
    head = (_ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens))
    tail = (_ptr(uniforms), float(temperature), B, k, V, _ptr(out_tokens), _ptr(num_accepted),
            _ptr(p_at_draft), _ptr(q_at_draft), _ptr(ws), ws.numel(), _stream(device, stream))
    if fn == "spec_verify_stochastic":
        st = lib.spec_verify_stochastic(*head, *tail)
    elif fn == "spec_verify_stochastic_ragged":
        st = lib.spec_verify_stochastic_ragged(*head, _ptr(draft_lens), *tail)
    elif fn == "spec_verify_stochastic_filtered":
        st = lib.spec_verify_stochastic_filtered(*head, *tail[:2], int(top_k), float(top_p),
                                                 float(min_p), *tail[2:])
    else:
        st = lib.spec_verify_stochastic_philox(*head, _ptr(draft_lens), int(seed) & (2**64 - 1),
                                               int(offset) & (2**64 - 1), *tail[1:])
    _lib.check(fn, st)
    return out_tokens, num_accepted


def spec_verify_stochastic(target_logits: torch.Tensor, draft_logits: torch.Tensor | None,
                           draft_tokens: torch.Tensor | None, uniforms: torch.Tensor,
                           temperature: float, *, out_tokens=None, num_accepted=None,
                           p_at_draft=None, q_at_draft=None, workspace=None, stream=None):
    """Stochastic verification; returns ``(out_tokens[B,k+1], num_accepted[B])``.

    ``p_at_draft`` / ``q_at_draft`` (float32 [B, k]), when given, receive the
    target and draft probabilities of each draft token.
    """
    return _stochastic("spec_verify_stochastic", target_logits, draft_logits, draft_tokens, None,
                       uniforms, temperature, out_tokens, num_accepted, p_at_draft, q_at_draft,
                       workspace, stream)


def spec_verify_stochastic_noalloc(target_logits: torch.Tensor,
                                   draft_logits: torch.Tensor | None,
                                   draft_tokens: torch.Tensor | None, uniforms: torch.Tensor,
                                   temperature: float, *, out_tokens, num_accepted,
                                   p_at_draft=None, q_at_draft=None, stream=None):
    """spec_verify_stochastic on the library's fixed per-GPU scratch array instead of a
    workspace: the call allocates nothing (the caller passes the outputs).  Calls
    that overlap in time on one GPU race on that array; shapes whose workspace
    exceeds ``_lib.NOALLOC_SCRATCH_BYTES`` raise (LIMIT_EXCEEDED)."""
    device = target_logits.device
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, k+1, V]")
    B, k1, V = target_logits.shape
    k = k1 - 1
    _dev(target_logits, "target_logits", device)
    if k > 0:
        _dev(draft_logits, "draft_logits", device, target_logits.dtype, (B, k, V))
        _dev(draft_tokens, "draft_tokens", device, torch.int32, (B, k))
    else:
        draft_logits = draft_tokens = None
    _dev(uniforms, "uniforms", device, torch.float32, (B, k + 1))
    _dev(out_tokens, "out_tokens", device, torch.int32, (B, k + 1))
    _dev(num_accepted, "num_accepted", device, torch.int32, (B,))
    for name, t in (("p_at_draft", p_at_draft), ("q_at_draft", q_at_draft)):
        if t is not None:
            _dev(t, name, device, torch.float32, (B, k))
    st = _lib.load().spec_verify_stochastic_noalloc(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens), _ptr(uniforms),
        float(temperature), B, k, V, _ptr(out_tokens), _ptr(num_accepted), _ptr(p_at_draft),
        _ptr(q_at_draft), _stream(device, stream))
    _lib.check("spec_verify_stochastic_noalloc", st)
    return out_tokens, num_accepted


def spec_verify_stochastic_ragged(target_logits: torch.Tensor, draft_logits: torch.Tensor | None,
                                  draft_tokens: torch.Tensor | None,
                                  draft_lens: torch.Tensor | None, uniforms: torch.Tensor,
                                  temperature: float, *, out_tokens=None, num_accepted=None,
                                  p_at_draft=None, q_at_draft=None, workspace=None,
                                  stream=None):
    """Stochastic verification with a draft length per request (int32 [B] on the
    device, clamped to [0, k]; None = k for all)."""
    return _stochastic("spec_verify_stochastic_ragged", target_logits, draft_logits,
                       draft_tokens, draft_lens, uniforms, temperature, out_tokens,
                       num_accepted, p_at_draft, q_at_draft, workspace, stream)


def spec_verify_stochastic_philox(target_logits: torch.Tensor,
                                  draft_logits: torch.Tensor | None,
                                  draft_tokens: torch.Tensor | None,
                                  draft_lens: torch.Tensor | None, seed: int, offset: int,
                                  temperature: float, *, out_tokens=None, num_accepted=None,
                                  p_at_draft=None, q_at_draft=None, workspace=None,
                                  stream=None):
    """Stochastic verification whose uniforms are Philox4x64-10 draws from
    ``(seed, offset)`` (draw i of request b: counter (offset, b, i // 4, 0), key
    (seed, 0), word i % 4, top 24 bits / 2^24)."""
    return _stochastic("spec_verify_stochastic_philox", target_logits, draft_logits,
                       draft_tokens, draft_lens, None, temperature, out_tokens, num_accepted,
                       p_at_draft, q_at_draft, workspace, stream, seed=seed, offset=offset)


def spec_verify_stochastic_filtered(target_logits: torch.Tensor,
                                    draft_logits: torch.Tensor | None,
                                    draft_tokens: torch.Tensor | None, uniforms: torch.Tensor,
                                    temperature: float, top_k: int = 0, top_p: float = 1.0,
                                    min_p: float = 0.0, *, out_tokens=None, num_accepted=None,
                                    p_at_draft=None, q_at_draft=None, workspace=None,
                                    stream=None):
    """Stochastic verification with top-k / top-p / min-p applied alike to every
    target and draft row (0 / 1.0 / 0.0 switch a filter off; top_p and min_p
    are passed as float32)."""
    return _stochastic("spec_verify_stochastic_filtered", target_logits, draft_logits,
                       draft_tokens, None, uniforms, temperature, out_tokens, num_accepted,
                       p_at_draft, q_at_draft, workspace, stream, top_k=top_k, top_p=top_p,
                       min_p=min_p)


def _greedy(fn, target_logits, draft_tokens, draft_lens, out_tokens, num_accepted, workspace,
            stream):
    device = target_logits.device
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, k+1, V]")
    B, k1, V = target_logits.shape
    k = k1 - 1
    _dev(target_logits, "target_logits", device)
    if k > 0:
        _dev(draft_tokens, "draft_tokens", device, torch.int32, (B, k))
    else:
        draft_tokens = None
    if draft_lens is not None:
        _dev(draft_lens, "draft_lens", device, torch.int32, (B,))
    if out_tokens is None:
        out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=device)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=device)
    _dev(out_tokens, "out_tokens", device, torch.int32, (B, k + 1))
    _dev(num_accepted, "num_accepted", device, torch.int32, (B,))
    nbytes = spec_verify_workspace_bytes(MODE_GREEDY, B, k + 1, V, dt)
    ws = _workspace(workspace, nbytes, device, stream)
    lib = _lib.load()
    tail = (B, k, V, _ptr(out_tokens), _ptr(num_accepted), _ptr(ws), ws.numel(),
            _stream(device, stream))
    if fn == "spec_verify_greedy":
        st = lib.spec_verify_greedy(_ptr(target_logits), dt, _ptr(draft_tokens), *tail)
    else:
        st = lib.spec_verify_greedy_ragged(_ptr(target_logits), dt, _ptr(draft_tokens),
                                           _ptr(draft_lens), *tail)
    _lib.check(fn, st)
    return out_tokens, num_accepted


def spec_verify_greedy(target_logits: torch.Tensor, draft_tokens: torch.Tensor | None, *,
                       out_tokens=None, num_accepted=None, workspace=None, stream=None):
    """Greedy verification; returns ``(out_tokens[B,k+1], num_accepted[B])``."""
    return _greedy("spec_verify_greedy", target_logits, draft_tokens, None, out_tokens,
                   num_accepted, workspace, stream)


def spec_verify_greedy_ragged(target_logits: torch.Tensor, draft_tokens: torch.Tensor | None,
                              draft_lens: torch.Tensor | None, *, out_tokens=None,
                              num_accepted=None, workspace=None, stream=None):
    """Greedy verification with a draft length per request (int32 [B] on the device)."""
    return _greedy("spec_verify_greedy_ragged", target_logits, draft_tokens, draft_lens,
                   out_tokens, num_accepted, workspace, stream)


def spec_verify_tree(target_logits: torch.Tensor, node_tokens: torch.Tensor,
                     paths: torch.Tensor, *, out_tokens=None, num_accepted=None,
                     best_path=None, accepted_nodes=None, workspace=None, stream=None):
    """Tree verification; returns ``(out_tokens[B,L], num_accepted[B], best_path[B],
    accepted_nodes[B,L])``."""
    device = target_logits.device
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3 or paths.dim() != 3:
        raise ValueError("target_logits must be [B, N+1, V] and paths [B, P, L]")
    B, N1, V = target_logits.shape
    _, P, L = paths.shape
    _dev(target_logits, "target_logits", device)
    _dev(node_tokens, "node_tokens", device, torch.int32, (B, N1))
    _dev(paths, "paths", device, torch.int32, (B, P, L))
    outs = []
    for name, t, shape in (("out_tokens", out_tokens, (B, L)),
                           ("num_accepted", num_accepted, (B,)),
                           ("best_path", best_path, (B,)),
                           ("accepted_nodes", accepted_nodes, (B, L))):
        if t is None:
            t = torch.empty(shape, dtype=torch.int32, device=device)
        outs.append(_dev(t, name, device, torch.int32, shape))
    nbytes = spec_verify_workspace_bytes(MODE_TREE, B, N1, V, dt)
    ws = _workspace(workspace, nbytes, device, stream)
    st = _lib.load().spec_verify_tree(
        _ptr(target_logits), dt, _ptr(node_tokens), _ptr(paths), B, N1 - 1, P, L, V,
        _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(outs[3]), _ptr(ws), ws.numel(),
        _stream(device, stream))
    _lib.check("spec_verify_tree", st)
    return tuple(outs)


GAVE_UP = -2  # num_accepted of a stochastic tree request whose split walk gave up waiting


def check_tree_stochastic_result(num_accepted: torch.Tensor) -> None:
    """Raise SpecVerifyError if a request of a stochastic tree call is marked as
    given up (num_accepted == -2: its workgroups stopped waiting for one another
    and its outputs are not valid).  Reads the tensor (synchronises with its
    stream when it lives on the GPU)."""
    bad = (num_accepted == GAVE_UP).nonzero().flatten().tolist()
    if bad:
        raise SpecVerifyError("spec_verify_tree_stochastic", _lib.HIP_ERROR,
                              f"the split walk of request(s) {bad[:8]} gave up waiting for "
                              "its workgroups (outputs not valid)")


def spec_verify_tree_stochastic(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                                node_tokens: torch.Tensor, paths: torch.Tensor,
                                uniforms: torch.Tensor, temperature: float, *, out_tokens=None,
                                num_accepted=None, accepted_nodes=None, workspace=None,
                                split=True, stream=None, check=True):
    """Stochastic tree verification (each accepted node's children tested in
    ascending order against the residual of their rejected siblings); returns
    ``(out_tokens[B,L], num_accepted[B], accepted_nodes[B,L])``.  ``uniforms``
    is float32 [B, N+1]: entry c-1 drives node c's test, entry N the final draw.
    With ``split`` (and a workspace, allocated here when not given) each
    request's walk may be shared by several workgroups; ``split=False`` passes
    no workspace (one workgroup per request).

    With ``check`` (the default) the call waits for its result and raises
    SpecVerifyError when a request's walk gave up (num_accepted == -2); a caller
    that reads num_accepted itself may pass ``check=False`` to stay
    asynchronous and call ``check_tree_stochastic_result`` when it does."""
    device = target_logits.device
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3 or paths.dim() != 3:
        raise ValueError("target_logits must be [B, N+1, V] and paths [B, P, L]")
    B, N1, V = target_logits.shape
    _, P, L = paths.shape
    _dev(target_logits, "target_logits", device)
    _dev(draft_logits, "draft_logits", device, target_logits.dtype, (B, N1, V))
    _dev(node_tokens, "node_tokens", device, torch.int32, (B, N1))
    _dev(paths, "paths", device, torch.int32, (B, P, L))
    _dev(uniforms, "uniforms", device, torch.float32, (B, N1))
    outs = []
    for name, t, shape in (("out_tokens", out_tokens, (B, L)),
                           ("num_accepted", num_accepted, (B,)),
                           ("accepted_nodes", accepted_nodes, (B, L))):
        if t is None:
            t = torch.empty(shape, dtype=torch.int32, device=device)
        outs.append(_dev(t, name, device, torch.int32, shape))
    ws = None
    if split:
        ws = _workspace(workspace, spec_verify_workspace_bytes(MODE_TREE_STOCHASTIC, B, N1, V, dt),
                        device, stream)
    st = _lib.load().spec_verify_tree_stochastic(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(node_tokens), _ptr(paths),
        _ptr(uniforms), float(temperature), B, N1 - 1, P, L, V, _ptr(outs[0]), _ptr(outs[1]),
        _ptr(outs[2]), _ptr(ws), 0 if ws is None else ws.numel(), _stream(device, stream))
    _lib.check("spec_verify_tree_stochastic", st)
    if check:
        check_tree_stochastic_result(outs[1])
    return tuple(outs)


def spec_verify_tree_stochastic_split(B: int, V: int, dtype: int = BF16) -> int:
    """Workgroups per request that spec_verify_tree_stochastic would use on the
    current device (1: not split; 0: arguments it would reject)."""
    return int(_lib.load().spec_verify_tree_stochastic_split(B, V, dtype))


def spec_verify_gather_rows(src: torch.Tensor, accepted_nodes: torch.Tensor,
                            num_accepted: torch.Tensor, dst: torch.Tensor, *, stream=None):
    """``dst[b, j] = src[b, accepted_nodes[b, j]]`` for ``j < num_accepted[b]`` (rows of
    any dtype and trailing shape, contiguous); other slots of ``dst`` are left
    as they are.  Returns ``dst``."""
    device = src.device
    if src.dim() < 2 or dst.dim() != src.dim() or dst.shape[2:] != src.shape[2:]:
        raise ValueError("src must be [B, N1, ...] and dst [B, L, ...] with the same row shape")
    if dst.dtype != src.dtype:
        raise TypeError("src and dst must have the same dtype")
    B, N1 = src.shape[:2]
    L = dst.shape[1]
    _dev(src, "src", device)
    _dev(dst, "dst", device, shape=(B, L) + tuple(src.shape[2:]))
    _dev(accepted_nodes, "accepted_nodes", device, torch.int32, (B, L))
    _dev(num_accepted, "num_accepted", device, torch.int32, (B,))
    row_bytes = src[0, 0].numel() * src.element_size() if src.numel() else 0
    st = _lib.load().spec_verify_gather_rows(_ptr(src), _ptr(dst), row_bytes,
                                             _ptr(accepted_nodes), _ptr(num_accepted), B, N1, L,
                                             _stream(device, stream))
    _lib.check("spec_verify_gather_rows", st)
    return dst
