"""The C API's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

hts_api.cpp is built for the host with both sanitizers, the kernel launchers replaced by
stand-ins that check what the host code hands them (tests/host_sanitize/launch_stubs.cpp); a
driver (abi_driver.cpp) calls every entry point with valid and invalid arguments, plans tile
indexes for random maps of every tile shape and element type (exactly sized output buffers), and
checks the per-thread error text from eight threads.  A planted caller mistake -- an index
buffer one record short -- must be reported as a heap overflow inside hts_pack_plan, which shows
that the sanitizer is live in this build.  The device code of hts_api.cpp (its scratch array) is
built without sanitizers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("asan")
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", f"-I{ROOT}/include",
              f"-I{ROOT}/tile_gemm_amd/csrc", f"-I{HERE}"]
    # host-side sanitizers only: each -fsanitize goes to the host compilation
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (f"{ROOT}/tile_gemm_amd/csrc/hts_api.cpp", f"{HERE}/launch_stubs.cpp", f"{HERE}/abi_driver.cpp"):
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *common, *san, "-x", "hip", "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(out / "abi_asan")
    # the link adds the host sanitizer runtimes; no GPU code is built with them
    r = subprocess.run([hipcc, "-fsanitize=address,undefined", "-fno-gpu-sanitize", "--offload-arch=gfx950", *objs,
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)


def test_every_entry_point_is_clean_under_asan_and_ubsan(driver):
    r = _run(driver)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert "expectations failed: 0, stub checks failed: 0" in r.stdout


def test_the_sanitizer_catches_a_planted_overflow(driver):
    r = _run(driver, "--plant-overflow")
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr and "hts_pack_plan" in r.stderr, r.stderr[-3000:]
