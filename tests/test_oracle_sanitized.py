"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle/moe_oracle.c is compiled with gcc's address and undefined-behaviour sanitizers (every
report fatal) and loaded in place of the normal build through MOE_ORACLE_LIB, with the
sanitizer runtime preloaded into the Python process that runs the five pin files.  Every
pin must pass with no report: no access outside a buffer, no signed overflow, no shift out
of range, no misaligned access.  A control copy with one planted off-by-one store (the
combine's output loop runs one element past the row) must stop with an AddressSanitizer
report, which shows the instrumentation is live in this setup.
"""
import importlib
import os
import subprocess
import sys

import pytest

obuild = importlib.import_module("oracle.build")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_f16_tokens.py", "tests/test_oracle_combine_quant.py",
             "tests/test_oracle_combine_scatter.py", "tests/test_oracle_quant_variants.py",
             "tests/test_oracle_pins.py"]
SAN_FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
             "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
# the gather combine's store of one output row, as the oracle writes it (its first
# occurrence; the int8 combine stores its rows the same way)
ROW_STORE = "for (int32_t h = 0; h < H; ++h) y_row[h] = f32_to_tok(c->token_dtype, acc[h]);"


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(src_path, out):
    subprocess.run(["gcc", *SAN_FLAGS, "-I", obuild.HERE, "-o", out, src_path, "-lm"],
                   check=True, capture_output=True)


def _run(lib, files, extra=()):
    env = dict(os.environ, MOE_ORACLE_LIB=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87",
               OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *extra, *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc's AddressSanitizer runtime is missing")
def test_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _build(obuild.SRC, lib)
    rc, out = _run(lib, PIN_FILES, extra=["-s"])
    assert rc == 0, (rc, out[-4000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc's AddressSanitizer runtime is missing")
def test_sanitizer_reports_a_planted_out_of_bounds_store(tmp_path):
    src = open(obuild.SRC).read()
    assert ROW_STORE in src, "the oracle's row store changed; update the control"
    bad = str(tmp_path / "oob.c")
    with open(bad, "w") as f:
        f.write(src.replace(ROW_STORE, ROW_STORE.replace("h < H", "h <= H"), 1))
    lib = str(tmp_path / "liboracle_oob.so")
    _build(bad, lib)
    # -s: the child's pytest must not hold its stderr, or the report dies with the process
    rc, out = _run(lib, ["tests/test_oracle_pins.py"], extra=["-s", "-k", "combine"])
    assert rc == 86 and "AddressSanitizer" in out, (rc, out[-4000:])
