"""Build tests/c/abi_layer (a plain C caller of the libssdscan C ABI, checked against the
fp64 oracle) into tests/c/_build.  Needs libssdscan.so and the oracle built first."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build", "abi_layer")
LIBDIRS = [os.path.join(ROOT, "chunked_linear_recurrence_amd", "_build"), os.path.join(ROOT, "oracle", "_build")]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(HERE, "abi_layer.c"), "-o", OUT,
           "-L", LIBDIRS[0], "-L", LIBDIRS[1], "-L", os.path.join(ROCM, "lib"),
           "-lssdscan", "-lssdoracle", "-lamdhip64", "-lm", "-pthread"]
    for d in LIBDIRS:
        cmd.append("-Wl,-rpath," + d.replace(ROOT, "$ORIGIN/../../.."))
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
