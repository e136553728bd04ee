"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds of the same sources run existing CPU tests in child processes
with the sanitizer runtime preloaded (LD_PRELOAD), any report aborting the
child:
  * the oracle (gcc, -fsanitize=address,undefined) runs its pins;
  * the library's host side (api.cpp: argument checks, workspace layouts,
    launch set-up; clang's sanitizers on the host pass only, kernels not
    instrumented and none launched here) runs the ABI host tests.
A planted heap overflow in a probe built the same way must abort its child
with an ASan report, which shows the checks are live in this set-up.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def gcc_runtimes():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"gcc has no {name}")
        libs.append(p)
    return ":".join(libs)


def clang_runtime():
    from mixture_experts_layer_logit_amd import build as b
    if not os.path.exists(b.HIPCC):
        pytest.skip("needs hipcc")
    rt = b.asan_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang's ASan runtime not found")
    return rt


def child(env_extra, argv, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    return subprocess.run(argv, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def pytest_child(env_extra, test_file):
    return child(env_extra, [sys.executable, "-m", "pytest", test_file, "-q", "-x", "-m", "not gpu",
                             "-p", "no:cacheprovider"])


def tail(r):
    return f"rc={r.returncode}\n--- stdout\n{r.stdout[-4000:]}\n--- stderr\n{r.stderr[-4000:]}"


def test_oracle_pins_under_sanitizers(tmp_path):
    import oracle
    pre = gcc_runtimes()
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = {"LD_PRELOAD": pre, "MOE_ORACLE_LIB": lib}
    r = child(env, [sys.executable, "-c", "import oracle; oracle._load(); "
                    f"print(any({lib!r} in l for l in open('/proc/self/maps')))"])
    assert r.returncode == 0 and r.stdout.strip() == "True", tail(r)
    r = pytest_child(env, "tests/test_oracle_pins.py")
    assert r.returncode == 0 and " passed" in r.stdout, tail(r)


def test_abi_host_under_sanitizers(tmp_path):
    from mixture_experts_layer_logit_amd import build as b
    rt = clang_runtime()
    try:
        lib = b.build_host_sanitized(str(tmp_path / "libmoe_san.so"))
    except FileNotFoundError as e:
        pytest.skip(f"kernel objects not built: {e}")
    env = {"LD_PRELOAD": rt, "MOE_LIB": lib}
    r = child(env, [sys.executable, "-c", "import mixture_experts_layer_logit_amd as m; m.load(); "
                    f"print(any({lib!r} in l for l in open('/proc/self/maps')))"])
    assert r.returncode == 0 and r.stdout.strip() == "True", tail(r)
    r = pytest_child(env, "tests/test_abi_host.py")
    assert r.returncode == 0 and " passed" in r.stdout, tail(r)


PROBE = r"""
#include <stdlib.h>
#ifdef __cplusplus
extern "C"
#endif
int probe_overflow(int n)
{
    int* a = (int*)malloc(n * sizeof(int));
    for (int i = 0; i <= n; ++i)  /* one element past the end */
        a[i] = i;
    int s = a[0];
    free(a);
    return s;
}
"""


def run_probe(lib, preload):
    return child({"LD_PRELOAD": preload},
                 [sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r}).probe_overflow(8)"], timeout=120)


def test_sanitizers_are_live_gcc(tmp_path):
    pre = gcc_runtimes()
    src = tmp_path / "probe.c"
    src.write_text(PROBE)
    lib = str(tmp_path / "probe_gcc.so")
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined", "-o", lib, str(src)],
                   check=True)
    r = run_probe(lib, pre)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, tail(r)


def test_sanitizers_are_live_hipcc(tmp_path):
    from mixture_experts_layer_logit_amd import build as b
    rt = clang_runtime()
    src = tmp_path / "probe.cpp"
    src.write_text(PROBE)
    obj, lib = str(tmp_path / "probe.o"), str(tmp_path / "probe_hip.so")
    san = []
    for check in ("address", "undefined"):
        san += ["-Xarch_host", "-fsanitize=" + check]
    subprocess.run([b.HIPCC, "-x", "hip", "-c", str(src), "-o", obj, "-O1", "-g", "-fPIC",
                    f"--offload-arch={b.ARCH}"] + san, check=True, capture_output=True)
    subprocess.run([b.HIPCC, "-shared", "-fPIC", f"--offload-arch={b.ARCH}", "-shared-libsan"] + san +
                   ["-o", lib, obj], check=True, capture_output=True)
    r = run_probe(lib, rt)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, tail(r)
