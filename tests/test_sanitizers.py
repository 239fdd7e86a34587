"""CPU sanitizer jobs (no GPU needed).

1. The oracle (oracle/moe_oracle.c) built with gcc under AddressSanitizer and
   UndefinedBehaviorSanitizer, driven by tests/sanitize/oracle_driver.c through
   every entry point and error path.
2. The host side of the C ABI: every translation unit of the library built
   with the sanitizers on the host half only (the device half is built
   without them, unoptimised, and never launched), driven by
   tests/sanitize/abi_driver.c through the host-only helpers and every
   validation path that returns before a launch.
Any report aborts the driver (no recovery), which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "moe_layer_align_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _layer_units():
    import moe_layer_align_amd.build as b  # the layer library's translation units, as built
    return [u[:-len(".hip")] for u in b.UNITS]


UNITS = _layer_units()
# sanitizers on the host half of each hipcc compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-4000:], res.stderr[-4000:])
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(ROOT, "oracle", "moe_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm"])
    res = _run([exe], env=dict(os.environ, OMP_NUM_THREADS="4"), timeout=300)
    assert "oracle sanitizer driver ok" in res.stdout


@pytest.mark.timeout(600)
def test_abi_host_paths_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    for u in UNITS:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xarch_device", "-O0",
               *HOST_SAN, *inc, "-c", os.path.join(CSRC, u + ".hip"), "-o", str(tmp_path / (u + ".o"))]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, "%s\n%s" % (" ".join(cmd), err[-4000:])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", *HOST_SAN, *inc, "-x", "c",
          os.path.join(HERE, "abi_driver.c"), "-x", "none", *[str(tmp_path / (u + ".o")) for u in UNITS],
          "-o", exe])
    res = _run([exe], timeout=300)
    assert "abi sanitizer driver ok" in res.stdout
