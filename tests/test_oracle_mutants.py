"""Planted mistakes in the oracle (CPU only).

Each mutant is a copy of oracle/moe_oracle.c with one plausible error -- a dropped term, a
wrong constant, a transposed index, a skipped rounding step, a reversed order -- compiled
with the oracle's own flags.  The oracle's pin suites then run against the copy (through
MOE_ORACLE_LIB) and must fail; a mutant that passes every pin is a gap in the pins.  The
unchanged copy, built and loaded the same way, must pass, which shows that the failures come
from the planted mistakes and not from the way the copies are loaded.
"""
import concurrent.futures
import importlib
import os
import subprocess
import sys

import pytest

obuild = importlib.import_module("oracle.build")   # the module, not the build() it exports

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fastest-failing files first: pytest stops at the first failure (-x)
PIN_FILES = ["tests/test_oracle_f16_tokens.py", "tests/test_oracle_combine_quant.py",
             "tests/test_oracle_combine_scatter.py", "tests/test_oracle_quant_variants.py",
             "tests/test_oracle_pins.py"]

_T = "float t = w * tok_to_f32(c->token_dtype, src[h]);"
_RQ = "double r = nearbyint(a / quantum) * quantum;"     # binary16, then E2M1
_NQ = "double n = nearbyint(a / quantum);"                # E4M3, then E5M2
_EMAX = "return ct == ORACLE_CODE_E4M3 ? 8 : ct == ORACLE_CODE_E5M2 ? 15 : 2;"
_ZE = "const int32_t zero_end = c->E + c->zero_expert_num;"   # the gather combine first

# (name, text in moe_oracle.c, replacement, which occurrence of the text); every mutant
# keeps its reads and writes inside the buffers, so it fails a pin rather than crashing
MUTANTS = [
    ("bf16 ties away from zero",
     "if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) keep += 1u;",
     "if (drop >= 0x8000u) keep += 1u;", 0),
    ("binary16 subnormal spacing halved",
     "quantum = ldexp(1.0, -24);", "quantum = ldexp(1.0, -25);", 0),
    ("E4M3 saturates one code low",
     "if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
     "if (a >= 448.0) return (uint8_t)(sign | 0x7D);", 0),
    ("E5M2 saturates one code low",
     "if (a >= 57344.0) return (uint8_t)(sign | 0x7B);",
     "if (a >= 57344.0) return (uint8_t)(sign | 0x7A);", 0),
    ("E2M1 saturates at 4",
     "if (isnan(v) || a >= 6.0) return (uint8_t)(sign | 0x7);",
     "if (isnan(v) || a >= 6.0) return (uint8_t)(sign | 0x6);", 0),
    ("int8 clamp at -128",
     "if (r < -127.0f) r = -127.0f;", "if (r < -128.0f) r = -128.0f;", 0),
    ("E8M0 bias 128",
     "return (uint8_t)((ex - 1) + 127);", "return (uint8_t)((ex - 1) + 128);", 0),
    ("MX shared exponent one high",
     "else se = ilog2_floor(amax) - code_emax(ct);",
     "else se = ilog2_floor(amax) - code_emax(ct) + 1;", 0),
    ("MX clip rounds an exact power of two up",
     "se = (m == 0.5f) ? ex - 1 : ex;", "se = (m == 1.0f) ? ex - 1 : ex;", 0),
    ("MX clip floor 1e-3 instead of 1e-4",
     "float c = amax > 1e-4f ? amax : 1e-4f;", "float c = amax > 1e-3f ? amax : 1e-3f;", 0),
    ("fp4 nibbles swapped",
     "q[h / 2] = (uint8_t)(one[h] | (one[h + 1] << 4));",
     "q[h / 2] = (uint8_t)(one[h + 1] | (one[h] << 4));", 0),
    ("dynamic scale as amax / max instead of 1 / dyn",
     "return 1.0f / dyn;", "return amax / code_max(ct);", 0),
    ("smooth-scale row read as a scalar",
     "else if (pre_len == H) f[h] = f[h] * pre[h];",
     "else if (pre_len == H) f[h] = f[h] * pre[0];", 0),
    ("per-group length 256 instead of 128",
     "for (int32_t g = 0; g * 128 < H; ++g) {\n"
     "            int32_t h1 = g * 128 + 128 < H ? g * 128 + 128 : H;\n"
     "            scales[g] = quant_dynamic(code_type, f, g * 128, h1, q);",
     "for (int32_t g = 0; g * 256 < H; ++g) {\n"
     "            int32_t h1 = g * 256 + 256 < H ? g * 256 + 256 : H;\n"
     "            scales[g] = quant_dynamic(code_type, f, g * 256, h1, q);", 0),
    ("routing ignores the mask",
     "if (!pair_active(c, mask, s, i, k) || e >= c->E) {", "if (e >= c->E) {", 0),
    ("expert_token_nums types swapped",
     "c->expert_token_nums_type == 0 ? run : per_expert;",
     "c->expert_token_nums_type == 1 ? run : per_expert;", 0),
    ("segment index transposed (source-major)",
     "int64_t flat = (int64_t)j * W + s;", "int64_t flat = (int64_t)s * L + j;", 0),
    ("combine drops the routed weight", _T, "float t = tok_to_f32(c->token_dtype, src[h]);", 0),
    ("copy expert unweighted", _T, "float t = tok_to_f32(c->token_dtype, src[h]);", 1),
    ("combine sums the picks in reverse order",
     "acc[h] = 0.0f;\n    for (int32_t k = 0; k < c->K; ++k) {",
     "acc[h] = 0.0f;\n    for (int32_t k = c->K - 1; k >= 0; --k) {", 0),
    ("combine int8 block scale by division",
     "float scale = amax * inv127;", "float scale = amax / 127.0f;", 0),
    ("combine int8 skips the binary16 step",
     "q[h] = oracle_int8_from_f16(oracle_f32_to_f16(v));", "q[h] = oracle_int8_from_f32(v);", 0),
    ("combine dequant block of 16",
     "out[h] = v * scales[h / 8];", "out[h] = v * scales[h / 16];", 0),
    ("scatter-back slot transposed",
     "size_t ep_offset = (size_t)i * K + k;", "size_t ep_offset = (size_t)k * c->BS + i;", 0),
    ("shared expert's term dropped", "if (shared_x) {", "if (0 && shared_x) {", 0),
    ("binary16 ties away from zero", _RQ, "double r = round(a / quantum) * quantum;", 0),
    ("E2M1 ties away from zero", _RQ, "double r = round(a / quantum) * quantum;", 1),
    ("E4M3 ties away from zero", _NQ, "double n = round(a / quantum);", 0),
    ("E5M2 ties away from zero", _NQ, "double n = round(a / quantum);", 1),
    ("int8 ties away from zero", "float r = nearbyintf(v);", "float r = roundf(v);", 0),
    ("NaN products encoded", "q[h] = isnan(v) ? 0 : encode(ct, v);", "q[h] = encode(ct, v);", 0),
    ("per-pick mask read per token",
     "return mask[((size_t)s * c->BS + i) * c->K + k] != 0;",
     "return mask[(size_t)s * c->BS + i] != 0;", 0),
    ("ordinals counted pick-major instead of token-major",
     "        for (int32_t i = 0; i < c->BS; ++i)\n"
     "            for (int32_t k = 0; k < c->K; ++k) {\n"
     "                size_t p = ((size_t)s * c->BS + i) * c->K + k;\n"
     "                int32_t e = expert_ids[p];\n"
     "                if (e < 0 || e >= id_end) return -1;",
     "        for (int32_t k = 0; k < c->K; ++k)\n"
     "            for (int32_t i = 0; i < c->BS; ++i) {\n"
     "                size_t p = ((size_t)s * c->BS + i) * c->K + k;\n"
     "                int32_t e = expert_ids[p];\n"
     "                if (e < 0 || e >= id_end) return -1;", 0),
    ("receiver windows not accumulated",
     "recv_offsets[r + 1] = recv_offsets[r] + run;", "recv_offsets[r + 1] = run;", 0),
    ("E5M2 emax 16", _EMAX, "return ct == ORACLE_CODE_E4M3 ? 8 : ct == ORACLE_CODE_E5M2 ? 16 : 2;", 0),
    ("E2M1 emax 1", _EMAX, "return ct == ORACLE_CODE_E4M3 ? 8 : ct == ORACLE_CODE_E5M2 ? 15 : 1;", 0),
    ("assist_info stores (s, k, i)",
     "assist_info[(size_t)row * 3 + 1] = i;\n                assist_info[(size_t)row * 3 + 2] = k;",
     "assist_info[(size_t)row * 3 + 1] = k;\n                assist_info[(size_t)row * 3 + 2] = i;", 0),
    ("zero experts combined as copy experts", _ZE, "const int32_t zero_end = c->E;", 0),
]


def _mutate(src, old, new, nth):
    at = -1
    for _ in range(nth + 1):
        at = src.find(old, at + 1)
        assert at >= 0, f"the oracle source no longer holds {old!r} (occurrence {nth})"
    return src[:at] + new + src[at + len(old):]


def _build(src_text, path):
    c_path = path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    # the oracle's flags, less -Werror: a mutant may leave a variable or parameter unused
    flags = [f for f in obuild.CFLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, "-I", obuild.HERE, "-o", path, c_path, "-lm"],
                   check=True, capture_output=True)


def _run_pins(lib, files):
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_mutant_texts_are_present():
    src = open(obuild.SRC).read()
    for name, old, new, nth in MUTANTS:
        assert _mutate(src, old, new, nth) != src, name


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(obuild.SRC).read()
    builds = {}
    for n, (name, old, new, nth) in enumerate(MUTANTS):
        lib = str(tmp_path / f"libmutant{n}.so")
        _build(_mutate(src, old, new, nth), lib)
        builds[name] = lib
    clean = str(tmp_path / "libclean.so")
    _build(src, clean)
    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as pool:
        futs = {name: pool.submit(_run_pins, lib, PIN_FILES) for name, lib in builds.items()}
        # the unchanged copy runs every pin file, so each caught mutant is caught by its
        # mutation and not by loading a copy through MOE_ORACLE_LIB
        clean_fut = pool.submit(_run_pins, clean, PIN_FILES)
        results = {name: f.result() for name, f in futs.items()}
        clean_rc, clean_out = clean_fut.result()
    assert clean_rc == 0, "the unchanged copy fails its pins:\n" + clean_out
    survivors = [name for name, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"mutants that pass every pin: {survivors}"
    odd = {name: out for name, (rc, out) in results.items() if rc != 1}
    assert not odd, f"mutants that did not end in a test failure: {odd}"
