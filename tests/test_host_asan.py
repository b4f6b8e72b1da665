"""The library's host code under AddressSanitizer (CPU only).

Every HIP source is compiled for gfx950 with the host half instrumented by ASan
(the device code is untouched), linked with a C driver that runs every entry
point's host-side validation, the workspace sizing and the kernel plan query over
a spread of shapes, and run.  Any out-of-bounds access, use after free or other
memory error in the host code aborts the driver with an ASan report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from routing_dispatch_expert_logits_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "asan", "abi_host_driver.c")
# host-only instrumentation: -Xarch_host in front of each sanitizer flag
ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(libbuild.HIPCC), reason="hipcc not available")
def test_abi_host_code_under_asan(tmp_path):
    objs, cmds = [], []
    flags = [f for f in libbuild.DEVICE_FLAGS if f != "-O3"] + ["-O1", "-g"]
    for src in libbuild.sources() + [DRIVER]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        lang = ["-x", "c"] if src.endswith(".c") else []
        base = [libbuild.HIPCC, *lang, "-I", os.path.join(libbuild.ROOT, "include")] if lang else \
               [libbuild.HIPCC, *flags]
        cmds.append(base + ASAN + ["-c", src, "-o", obj])
    with ThreadPoolExecutor(8) as pool:
        for r in pool.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds):
            assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_host_driver")
    r = subprocess.run([libbuild.HIPCC, f"--offload-arch={libbuild.ARCH}", *ASAN, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "all checks passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
