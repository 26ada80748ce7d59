"""The library's host-only entry points (configuration checks, window and pass plans, the int4
quantiser, conditioning lengths, create's blob-size rejection) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU by tests/sanitize/host_driver.cpp.  The API source
(which holds no kernels) is linked with launcher stubs that refuse any launch; the sanitizers
instrument host code only."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
COMMON = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_entry_points_under_asan_and_ubsan(tmp_path):
    src = {"api": os.path.join(ROOT, "audio_encoder_amd", "csrc", "ae_api.hip"),
           "stubs": os.path.join(ROOT, "tests", "sanitize", "launch_stubs.hip"),
           "driver": os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")}
    objs = []
    for name, path in src.items():
        obj = str(tmp_path / f"{name}.o")
        lang = ["-x", "hip"] if path.endswith(".hip") else []
        run([HIPCC, *COMMON, *SAN, *lang, "-c", path, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_driver")
    run([HIPCC, *SAN, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = run([exe], env=env, timeout=300)
    assert "all checks passed" in r.stdout
