"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; the gfx950 code is not instrumented).

Each run is a child process with the sanitizer runtime preloaded: the oracle
built by gcc with -fsanitize=address,undefined (gcc's runtime) runs its pin
tests, and the HIP library built with the host-only sanitizer flags (clang's
runtime) runs the C-ABI host tests.  The two runtimes are never mixed in one
process.  A sanitizer report aborts the child (recovery off), which fails the
test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = ["test_oracle_codecs.py", "test_oracle_attention.py", "test_oracle_meta.py",
                "test_oracle_page_table.py", "test_oracle_prologue.py", "test_oracle_qk_norm.py",
                "test_oracle_sparse.py", "test_synth.py"]

CANARY = ("import ctypes, sys; sys.path.insert(0, {root!r}); "
          "ctypes.CDLL(None)['__asan_init']; "  # the runtime is in the process
          "{check}")


def _run(env_extra, args, check):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    c = subprocess.run([sys.executable, "-c", CANARY.format(root=ROOT, check=check)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert c.returncode == 0, c.stdout + c.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *args], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout


def test_oracle_under_address_and_undefined_behaviour_sanitizers():
    import oracle
    oracle.build(sanitize=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.exists(libasan), libasan
    check = ("import oracle; L = oracle.lib(); "
             "assert L._name.endswith('liboracle_san.so'), L._name")
    _run({"ORACLE_SANITIZE": "1", "LD_PRELOAD": libasan},
         [os.path.join("tests", t) for t in ORACLE_TESTS], check)


def test_host_library_under_address_and_undefined_behaviour_sanitizers():
    from attention_decode_qk_amd import build
    lib = build.build(force=False, sanitize=True)
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    check = ("import attention_decode_qk_amd as ga; L = ga.lib(); "
             "assert L._name.endswith('libmi355x_gated_attn_san.so'), L._name")
    _run({"MI355X_GA_LIB": lib, "LD_PRELOAD": rts[-1]},
         [os.path.join("tests", "test_abi_host.py")], check)
