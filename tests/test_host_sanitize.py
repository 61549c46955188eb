"""The C ABI's host logic under AddressSanitizer and UBSan (no GPU).

Builds tests/host_abi_sanitize.cpp against the library sources with the
sanitizers on the host code only: abi.cpp and the driver through hipcc with
each sanitizer flag behind -Xarch_host (the .hip sources keep their gfx950
device code, unsanitized, though no kernel is launched here), and the link
done by g++. The driver calls the host-only entry points and the argument checks of the GPU
entry points on exactly-sized heap buffers; any out-of-bounds access or
undefined behaviour stops it with a report.
"""

import os
import shutil
import subprocess

import pytest

from decode_attention_slot_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_slot_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
# the library's device sources, as its build lists them
HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]
# each sanitizer flag applies to host code only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and shutil.which("g++")),
                    reason="needs hipcc and g++")
def test_host_abi_under_address_and_ub_sanitizers(tmp_path):
    common = ["-O1", "-g", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}",
              f"-I{CSRC}"]
    hip = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops"]
    jobs = [(os.path.join(CSRC, "abi.cpp"), []),
            (os.path.join(ROOT, "tests", "host_abi_sanitize.cpp"), [])] + \
        [(os.path.join(CSRC, h), hip) for h in HIP_SOURCES]
    objs, procs = [], []
    for src, extra in jobs:  # compiled side by side
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, *common, *extra, *SAN, "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{' '.join(cmd)}\n{out}\n{err}"
    exe = str(tmp_path / "host_abi_sanitize")
    run(["g++", "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = run([exe], env=env, timeout=300)
    assert r.stdout.startswith("ok "), r.stdout + r.stderr
