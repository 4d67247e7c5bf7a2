"""Build tests/c_abi/c_abi_example (plain C99, gcc) against the in-tree
libmoe_route.so and the oracle's library.  Test infrastructure."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "c_abi_example")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(HERE, "c_abi_example.c"), "-o", EXE,
           "-L", os.path.join(ROOT, "combine_moe_route_amd"), "-lmoe_route",
           "-L", os.path.join(ROOT, "oracle"), "-lmoe_oracle",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../combine_moe_route_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return EXE


if __name__ == "__main__":
    print(build())
