"""ctypes loader for ``libspec_verify.so`` (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspec_verify.so")

# Stable enums, same values as include/spec_verify.h.
F32, BF16 = 0, 1
MODE_STOCHASTIC, MODE_GREEDY, MODE_TREE, MODE_STOCHASTIC_FILTERED, MODE_TREE_STOCHASTIC = range(5)
OK, INVALID_ARGUMENT, UNSUPPORTED_DTYPE, WORKSPACE_TOO_SMALL, LIMIT_EXCEEDED, HIP_ERROR = range(6)
NOALLOC_SCRATCH_BYTES = 8 << 20  # SPEC_VERIFY_NOALLOC_SCRATCH_BYTES
SCHEDULE_AUTO, SCHEDULE_TWO_KERNELS, SCHEDULE_SELF_COMPUTE, SCHEDULE_INTERLEAVED = 0, 1, 2, 3

EXPORTED = (
    "spec_verify_version",
    "spec_verify_status_string",
    "spec_verify_workspace_bytes",
    "spec_verify_workspace_init",
    "spec_verify_profile_events",
    "spec_verify_set_schedule",
    "spec_verify_stochastic",
    "spec_verify_stochastic_ragged",
    "spec_verify_stochastic_noalloc",
    "spec_verify_stochastic_philox",
    "spec_verify_stochastic_filtered",
    "spec_verify_greedy",
    "spec_verify_greedy_ragged",
    "spec_verify_tree",
    "spec_verify_tree_stochastic",
    "spec_verify_tree_stochastic_split",
    "spec_verify_debug_tree_spin_limit",
    "spec_verify_debug_spin_limit",
    "spec_verify_gather_rows",
)

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} (status {status})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.spec_verify_version.argtypes = []
    lib.spec_verify_version.restype = I
    lib.spec_verify_status_string.argtypes = [I]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.spec_verify_workspace_bytes.restype = Z
    lib.spec_verify_workspace_init.argtypes = [P, Z, P]
    lib.spec_verify_workspace_init.restype = I
    lib.spec_verify_profile_events.argtypes = [P, I]
    lib.spec_verify_profile_events.restype = I
    lib.spec_verify_set_schedule.argtypes = [I]
    lib.spec_verify_set_schedule.restype = I
    lib.spec_verify_stochastic.argtypes = [P, P, I, P, P, ctypes.c_float, I, I, I, P, P, P, P,
                                           P, Z, P]
    lib.spec_verify_stochastic.restype = I
    lib.spec_verify_stochastic_ragged.argtypes = [P, P, I, P, P, P, ctypes.c_float, I, I, I, P,
                                                  P, P, P, P, Z, P]
    lib.spec_verify_stochastic_ragged.restype = I
    lib.spec_verify_stochastic_noalloc.argtypes = [P, P, I, P, P, ctypes.c_float, I, I, I, P, P,
                                                   P, P, P]
    lib.spec_verify_stochastic_noalloc.restype = I
    U64 = ctypes.c_uint64
    lib.spec_verify_stochastic_philox.argtypes = [P, P, I, P, P, U64, U64, ctypes.c_float, I, I,
                                                  I, P, P, P, P, P, Z, P]
    lib.spec_verify_stochastic_philox.restype = I
    F = ctypes.c_float
    lib.spec_verify_stochastic_filtered.argtypes = [P, P, I, P, P, F, I, F, F, I, I, I, P, P, P,
                                                    P, P, Z, P]
    lib.spec_verify_stochastic_filtered.restype = I
    lib.spec_verify_greedy.argtypes = [P, I, P, I, I, I, P, P, P, Z, P]
    lib.spec_verify_greedy.restype = I
    lib.spec_verify_greedy_ragged.argtypes = [P, I, P, P, I, I, I, P, P, P, Z, P]
    lib.spec_verify_greedy_ragged.restype = I
    lib.spec_verify_tree.argtypes = [P, I, P, P, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.spec_verify_tree.restype = I
    lib.spec_verify_tree_stochastic.argtypes = [P, P, I, P, P, P, ctypes.c_float, I, I, I, I, I,
                                                P, P, P, P, Z, P]
    lib.spec_verify_tree_stochastic_split.argtypes = [I, I, I]
    lib.spec_verify_tree_stochastic_split.restype = I
    lib.spec_verify_debug_tree_spin_limit.argtypes = [I]
    lib.spec_verify_debug_tree_spin_limit.restype = I
    lib.spec_verify_debug_spin_limit.argtypes = [I]
    lib.spec_verify_debug_spin_limit.restype = I
    lib.spec_verify_tree_stochastic.restype = I
    lib.spec_verify_gather_rows.argtypes = [P, P, Z, P, P, I, I, I, P]
    lib.spec_verify_gather_rows.restype = I
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != OK:
        msg = load().spec_verify_status_string(status).decode()
        raise SpecVerifyError(fn, status, msg)
