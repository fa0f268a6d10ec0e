"""The CPU oracle and the library's host-side validation under AddressSanitizer
and UndefinedBehaviorSanitizer.  Nothing here launches a kernel: the oracle is
plain C, and every library call in the ABI suite is rejected on the host."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "spec_verify_oracle.c")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "oracle_edges.c")
CSRC = os.path.join(ROOT, "draft_token_verification_verify_amd", "csrc")
REPORT_MARKERS = ("AddressSanitizer", "LeakSanitizer", "runtime error:")
SAN_ENV = {"ASAN_OPTIONS": "halt_on_error=1:detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_sanitized(sources, out):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    cmd = [gcc, "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
           "-fsanitize=address,undefined", *sources, "-lm", "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def _run(cmd, env_extra=None, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra or {})
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True,
                          timeout=timeout)


def test_oracle_edge_shapes_are_clean(tmp_path):
    """Every oracle entry point on k = 0, V = 1, N = 0, P = 0, B = 0 and ragged,
    out-of-range and partly unused inputs, in exactly sized heap buffers: no
    sanitizer report, no leak, the expected statuses."""
    exe = _gcc_sanitized([ORACLE_SRC, DRIVER], str(tmp_path / "oracle_edges"))
    r = _run([exe])
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert not any(m in out for m in REPORT_MARKERS), out[-4000:]
    assert "oracle edge shapes: ok" in r.stdout


def test_a_planted_overread_is_reported(tmp_path):
    """The same build with one loop of the oracle's softmax running one element
    past the row: the sanitizer must stop the driver (so the clean run above
    means something)."""
    src = open(ORACLE_SRC).read()
    needle = ("    for (int j = 0; j < V; ++j) {\n"
              "        double z = logit_at(logits, dtype, row_offset + (size_t)j) / temperature;")
    assert src.count(needle) == 1
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(needle, needle.replace("j < V", "j <= V")))
    exe = _gcc_sanitized([str(mutant), DRIVER], str(tmp_path / "oracle_mutant"))
    r = _run([exe])
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stderr[-4000:]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_sanitized_library(out_dir):
    """The library with its host code instrumented (device code as usual; it is
    never launched here)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
    procs = [subprocess.Popen([hipcc, *flags, "-c", s, "-o", o], stdout=subprocess.DEVNULL,
                              stderr=subprocess.PIPE) for s, o in zip(srcs, objs)]
    for p, s in zip(procs, srcs):
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, f"{s}: {err.decode()[-2000:]}"
    lib = os.path.join(out_dir, "libspec_verify_sanitized.so")
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC",
            "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-shared-libsan", *objs, "-o", lib]
    subprocess.run(link, check=True, capture_output=True)
    return lib


def test_host_validation_is_clean(tmp_path):
    """The C-ABI suite (every entry point's rejection paths, workspace sizing,
    the schedule and testing hooks) against the library built with its host
    code under ASan and UBSan: it passes with no sanitizer report."""
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime not found")
    lib = _build_sanitized_library(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle_" in syms, "host code not instrumented"
    script = ("import sys\n"
              "from draft_token_verification_verify_amd import _lib\n"
              "_lib.LIB_PATH = sys.argv[1]\n"
              "import pytest\n"
              "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n")
    # The interpreter itself is not instrumented: leak reports would name its
    # own allocations, so leak checking is off here (it is on for the oracle).
    r = _run([sys.executable, "-c", script, lib],
             env_extra={"LD_PRELOAD": rt, "ASAN_OPTIONS": "halt_on_error=1:detect_leaks=0"},
             timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, out[-4000:]
    assert not any(m in out for m in REPORT_MARKERS), out[-4000:]
