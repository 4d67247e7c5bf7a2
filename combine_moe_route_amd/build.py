"""Build libmoe_route.so (the HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libmoe_route.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fvisibility=hidden",
    # no packed fp32 instructions: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _run(cmds: list[list[str]], jobs: int) -> str:
    """Run the commands, at most `jobs` at a time; raise on the first failure."""
    log, pending, running = [], list(cmds), []
    while pending or running:
        while pending and len(running) < jobs:
            cmd = pending.pop(0)
            running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                  text=True)))
        cmd, proc = running.pop(0)
        out, _ = proc.communicate()
        if proc.returncode != 0:
            for _, other in running:
                other.wait()
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
        log.append(out)
    return "".join(log)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source under csrc/ (one hipcc per file, in parallel) and
    link them into combine_moe_route_amd/libmoe_route.so."""
    jobs = jobs or max(1, min(len(sources()), os.cpu_count() or 1, 8))
    with tempfile.TemporaryDirectory(prefix="moe_route_build_") as tmpdir:
        objs, compiles = [], []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            compiles.append([hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        out = _run(compiles, jobs)
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        out += _run([[hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]], 1)
    if verbose and out:
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
