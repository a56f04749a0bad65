"""Builds tests/c_abi/abi_demo (plain C11 against include/moe_dc.h, libmoe_dc.so and the HIP
runtime), next to its source.  Test infrastructure: the GPU tests run the binary."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "abi_demo")
LIBDIR = os.path.join(ROOT, "combine_quant_amd")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "abi_demo.c"), "-o", BIN + ".tmp",
           "-L" + LIBDIR, "-lmoe_dc", "-Wl,-rpath," + LIBDIR, "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
