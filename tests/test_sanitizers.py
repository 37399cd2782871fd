"""The oracle and the host validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; no GPU code is instrumented).

* The oracle's C source is built with gcc's ``-fsanitize=address,undefined``
  and the oracle's own pins (token recurrence, gated-decay branch, backward)
  run against that build in a child process with the sanitizer runtimes
  preloaded (the interpreter itself is not instrumented).
* The C-ABI validation layer (``gdn_api.hip``) is built with its host code
  instrumented (``-Xarch_host`` before each sanitizer flag, so the device code
  is built as usual) and linked with the other objects of the library; the
  CPU ABI tests then call every entry point with fake device addresses, which
  the layer must reject or accept without touching them.
Each child must pass and print no sanitizer report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def run_child(code, env):
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=900)
    out = res.stdout + res.stderr
    print(out[-3000:])
    assert res.returncode == 0, "sanitized run failed"
    for r in REPORTS:
        assert r not in out, f"sanitizer report: {r}"
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = gcc_runtime("libasan.so"), gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libgdn_oracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                    "-o", lib, os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               OMP_NUM_THREADS="4")
    code = ("import sys, pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'tests/test_oracle_pins.py', 'tests/test_oracle_pins_decay.py', 'tests/test_oracle_backward.py', "
            "'-k', 'not mutant and not planted']))")
    out = run_child(code, env)
    assert " passed" in out


def test_validation_layer_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    objs = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o")) if not o.endswith("gdn_api.hip.o")]
    if not (hipcc and rt and objs):
        pytest.skip("needs hipcc, clang's ASan runtime and a built library (_build/*.o)")
    csrc = os.path.join(ROOT, "hybrid_linear_attention_gated_amd", "csrc")
    obj, lib = str(tmp_path / "gdn_api_asan.o"), str(tmp_path / "libgdn_asan.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                    "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(csrc, "gdn_api.hip"), "-o", obj],
                   check=True, capture_output=True)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-shared-libsan", "-o", lib, obj,
                    *objs], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0")
    code = ("import sys; sys.path.insert(0, 'tests'); import hybrid_linear_attention_gated_amd as gdn; "
            f"gdn.LIB_PATH = {lib!r}; import pytest; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))")
    out = run_child(code, env)
    assert " passed" in out
