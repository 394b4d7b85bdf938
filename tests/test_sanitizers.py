"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle is rebuilt with ``-fsanitize=address,undefined`` (gcc) and the
  oracle's pin tests run against that build in a child interpreter with gcc's
  runtimes preloaded: every oracle function the pins reach runs instrumented.
* libsqf's C-ABI host code (sqf_api.hip: argument checks, workspace sizing,
  launch set-up) is rebuilt with host-side ASan + UBSan (device code as in the
  product library) and the CPU ABI tests run against it with clang's runtime
  preloaded.  Nothing here touches a GPU.
Any sanitizer report aborts the child, so a non-zero exit fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_child(args, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def _exports_sanitizer_hooks(lib):
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    return "__asan_" in out and "__ubsan_" in out


def test_oracle_pins_under_asan_ubsan():
    import oracle

    lib = oracle.build(force=True, sanitize=True)
    assert _exports_sanitizer_hooks(lib)
    env = {"LD_PRELOAD": _gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"),
           "SQF_ORACLE_LIBRARY": lib}
    # the child really loads the sanitizer build
    r = _run_child(["-c", "import oracle; oracle._load(); print(oracle._lib._name)"], env)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stdout + r.stderr
    r = _run_child(["-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p", "no:cacheprovider"], env)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout


def test_abi_host_code_under_asan_ubsan():
    from outlier_split_mixed_amd import build as b

    if len(glob.glob(os.path.join(b.BUILD, "*.hip.o"))) != len(glob.glob(os.path.join(b.CSRC, "*.hip"))):
        pytest.skip("the kernel objects of a library build are not in _build/")
    lib = b.build_host_sanitized()
    assert _exports_sanitizer_hooks(lib)
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    env = {"LD_PRELOAD": rts[0], "SQF_LIBRARY": lib}
    r = _run_child(["-c", "from outlier_split_mixed_amd import sqf; print(sqf.LIB_PATH)"], env)
    assert r.returncode == 0 and r.stdout.strip().endswith(lib), r.stdout + r.stderr
    r = _run_child(["-m", "pytest", "tests/test_abi_cpu.py", "-q", "-x", "-p", "no:cacheprovider"], env)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout
