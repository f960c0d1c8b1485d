"""CPU: the library's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer (device code unchanged), driven through every size
query over a grid of valid and invalid configurations and through the
argument-error paths of every entry point (tests/host_sanitize/driver.cpp).
Nothing reaches the GPU.  The build goes to _build/sanitize and is reused
while no source is newer than it."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from scale_gla_layer_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")
# host-side instrumentation only: every sanitizer flag goes to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    try:
        return libbuild.hipcc()
    except RuntimeError:
        return None


def _sources():
    return [os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES]


def _newest_input():
    files = _sources() + [DRIVER, os.path.join(ROOT, "include", "msgla.h")]
    csrc = libbuild.CSRC
    files += [os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hpp", ".h"))]
    return max(os.path.getmtime(f) for f in files)


def _compile(args):
    src, obj, extra = args
    cmd = [_hipcc(), *libbuild.FLAGS, *HOST_SAN, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{res.stdout}{res.stderr}")
    return obj


def _build() -> str:
    exe = os.path.join(OUT, "driver")
    if os.path.exists(exe) and os.path.getmtime(exe) > _newest_input():
        return exe
    os.makedirs(OUT, exist_ok=True)
    jobs = []
    for src in _sources():
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        jobs.append((src, obj, ["-x", "hip"] if src.endswith(".cpp") else []))
    jobs.append((DRIVER, os.path.join(OUT, "driver_main.o"), []))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    tmp = exe + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={libbuild.ARCH}", *HOST_SAN, *objs, "-o", tmp, *libbuild.LIBS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, exe)
    return exe


@pytest.mark.skipif(_hipcc() is None or shutil.which("ld") is None, reason="needs hipcc")
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text
    assert "runtime error" not in text and "Sanitizer" not in text, text
    assert "failures 0" in res.stdout, text
