"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/sanitize/abi_validation_main.cpp calls every entry point with malformed arguments and
checks the returned codes.  It is linked with the library's host code built here with
-fsanitize=address,undefined on the host pass (mars_api.cpp and the kernel sources' launchers;
the device code is built as usual).  The process sees no GPU, so a call that passes validation
stops at its launch with MARS_EHIP.  Any sanitizer report or unexpected code fails the test."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_mask_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["mars_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "decode.hip", "accept.hip", "mask_kernels.hip",
           "kv_commit.hip", "shifted_ce.hip"]
# Each sanitizer flag goes to the host pass only.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_asan_ubsan(tmp_path):
    def compile_one(src):
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        r = subprocess.run([HIPCC, *FLAGS, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stdout}\n{r.stderr}"
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "sanitize",
                                                                    "abi_validation_main.cpp")]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_validation")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, f"link:\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-4000:], r.stderr[-4000:])
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert "0 failure(s)" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
