"""Ahead-of-time build of the gfx950 HIP libraries: the layer
(libmoe_mi355x.so) and the measurement probes (libmoe_probes.so).

Compiles the translation units under moe_layer_align_amd/csrc with hipcc for
gfx950, in parallel, and links them into the package directory.  Every unit
carries its own code object (no relocatable device code).  Packed-fp32
instructions are disabled (the compiler may otherwise fuse fp32 pairs into
v_pk_* forms).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
UNITS = ["moe_api.hip", "launch_decode_bf16.hip", "launch_decode_fp8.hip", "launch_decode_fp8_static.hip",
         "launch_prefill.hip", "launch_layer1.hip", "launch_down_token.hip"]
LIB = os.path.join(PKG, "libmoe_mi355x.so")
PROBE_UNITS = ["probes.hip"]
PROBE_LIB = os.path.join(PKG, "libmoe_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def _compile_link(units, lib, inc, verbose, extra, tmpdir, tag):
    """Start the compiles of `units`; returns a function that waits for them
    and links `lib`."""
    procs = []
    for unit in units:
        obj = os.path.join(tmpdir, tag + "_" + unit.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *extra, *inc, "-c", os.path.join(CSRC, unit), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((unit, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))

    def finish():
        objs, failed = [], []
        for unit, obj, p in procs:
            _, err = p.communicate()
            err = _clean(err)
            if p.returncode != 0:
                failed.append(unit)
                sys.stderr.write(err + "\n")
            elif verbose and err.strip():
                sys.stderr.write(err + "\n")
            objs.append(obj)
        if failed:
            raise RuntimeError("hipcc failed on %s" % ", ".join(failed))
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(_clean(res.stderr) + "\n")
            raise RuntimeError("hipcc link failed (%d)" % res.returncode)
        os.replace(tmp, lib)
    return finish


def build(verbose: bool = False, extra=()) -> str:
    """Build both libraries (all units compile in parallel); returns the
    layer library's path."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        layer = _compile_link(UNITS, LIB, inc, verbose, extra, tmpdir, "layer")
        probes = _compile_link(PROBE_UNITS, PROBE_LIB, inc, verbose, extra, tmpdir, "probes")
        layer()
        probes()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
