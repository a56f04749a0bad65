"""The C ABI from plain C: include/moe_dc.h compiles as strict C11, and (on a GPU) a C
program linked only against libmoe_dc.so and the HIP runtime runs dispatch and all three
combines (gather, scatter-back, int8 block-quantized) and checks them with invariants
(tests/c_abi/abi_demo.c)."""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DEMO = os.path.join(HERE, "c_abi", "abi_demo")


def test_header_is_strict_c11():
    src = "#include \"moe_dc.h\"\nint main(void) { moe_dc_config c = {0}; (void)c; return 0; }\n"
    subprocess.run(["gcc", "-std=c11", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-fsyntax-only", "-I" + os.path.join(ROOT, "include"), "-x", "c", "-"],
                   input=src.encode(), check=True)


def test_demo_is_built():
    assert os.path.exists(DEMO), "tests/c_abi/abi_demo is built by __graft_entry__.build()"


@pytest.mark.gpu
@pytest.mark.parametrize("shape", ["8 32 8 7168 8 200", "16 256 512 7168 8 20",
                                   "2 8 16 1030 2 50"])
def test_plain_c_consumer(shape):
    r = subprocess.run([DEMO, *shape.split()], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    m = re.search(r"ok routed=(\d+) step_us=([\d.]+)", r.stdout)
    W, E, BS, H, K, _ = map(int, shape.split())
    assert m and int(m.group(1)) == W * BS * K
