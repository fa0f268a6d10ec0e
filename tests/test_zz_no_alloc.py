"""The allocation-free stochastic call (spec_verify_stochastic_noalloc) against the
workspace-taking one: both run the same kernels, so their outputs must agree
bit for bit.  Two calls in a row, the second on a smaller input; the fixed
scratch array keeps the first call's state, which the library leaves zero."""
import ctypes

import numpy as np
import pytest
import torch

from draft_token_verification_verify_amd import _lib
from draft_token_verification_verify_amd import workloads as wl
import draft_token_verification_verify_amd as sv

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _outputs(case):
    dev = torch.device("cuda", 0)
    return dict(out=torch.full((case.B, case.k + 1), -7, dtype=torch.int32, device=dev),
                acc=torch.full((case.B,), -7, dtype=torch.int32, device=dev),
                p=torch.full((case.B, case.k), -1.0, dtype=torch.float32, device=dev),
                q=torch.full((case.B, case.k), -1.0, dtype=torch.float32, device=dev))


def _run_both(case):
    t = wl.to_device(case.target, case.dtype)
    d = wl.to_device(case.draft, case.dtype)
    x = wl.to_device(case.draft_tokens.astype(np.int32))
    u = wl.to_device(case.uniforms.astype(np.float32))
    dt = _lib.BF16 if case.dtype == "bf16" else _lib.F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = _lib.load()

    # the allocation-free call, through the C ABI
    na = _outputs(case)
    print(f"noalloc: {case.name}", flush=True)
    st = lib.spec_verify_stochastic_noalloc(
        _ptr(t), _ptr(d), dt, _ptr(x), _ptr(u), ctypes.c_float(case.temperature), case.B,
        case.k, case.V, _ptr(na["out"]), _ptr(na["acc"]), _ptr(na["p"]), _ptr(na["q"]), stream)
    assert st == _lib.OK, lib.spec_verify_status_string(st)

    # the workspace-taking call, with a fresh zeroed workspace of its own size
    ref = _outputs(case)
    nbytes = lib.spec_verify_workspace_bytes(_lib.MODE_STOCHASTIC, case.B, case.k + 1, case.V, dt)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    st = lib.spec_verify_stochastic(
        _ptr(t), _ptr(d), dt, _ptr(x), _ptr(u), ctypes.c_float(case.temperature), case.B,
        case.k, case.V, _ptr(ref["out"]), _ptr(ref["acc"]), _ptr(ref["p"]), _ptr(ref["q"]),
        _ptr(ws), nbytes, stream)
    assert st == _lib.OK, lib.spec_verify_status_string(st)
    torch.cuda.synchronize()
    for key in ("out", "acc"):
        assert torch.equal(na[key], ref[key]), f"{case.name}: {key} differs"
    for key in ("p", "q"):  # same kernels, same arithmetic: the same bits
        assert torch.equal(na[key].view(torch.int32), ref[key].view(torch.int32)), \
            f"{case.name}: {key} differs"
    assert int((ws != 0).sum()) == 0, "the workspace-taking call left its workspace dirty"
    return na


def test_noalloc_matches_the_workspace_call_twice():
    big = wl.c3(0, B=32)  # B=32, k=3, V=128256 bf16, T=0.8
    small = wl.c1(1)      # B=1, k=3, V=1000 fp32, then a smaller call on the same scratch
    _run_both(big)
    _run_both(small)
    _run_both(big)


def test_noalloc_rejects_an_oversized_shape_before_launching():
    lib = _lib.load()
    dev = torch.device("cuda", 0)
    out = torch.full((512, 6), -7, dtype=torch.int32, device=dev)
    acc = torch.full((512,), -7, dtype=torch.int32, device=dev)
    fake = ctypes.c_void_p(0x1000)  # never read: the host check fails first
    st = lib.spec_verify_stochastic_noalloc(fake, fake, _lib.F32, fake, fake, ctypes.c_float(1.0),
                                            512, 5, 151936, _ptr(out), _ptr(acc), None, None,
                                            None)
    assert st == _lib.LIMIT_EXCEEDED
    torch.cuda.synchronize()
    assert int((out != -7).sum()) == 0 and int((acc != -7).sum()) == 0
