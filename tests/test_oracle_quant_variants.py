"""Pins of the oracle's further quantization variants, against what the pages and the
number formats fix, computed independently of the oracle's C code:

  * E5M2 decoding against numpy's IEEE half precision (E5M2 is the upper byte of a binary16
    pattern), E5M2 encoding against a nearest-value search over the format's values and,
    in range, against torch's float8_e5m2 cast;
  * the int8 cast at its rounding ties and saturation points;
  * E8M0 bytes of every power of two the MX scales can take;
  * the per-mode code types and scale counts of the low_latency_dispatch constraints;
  * static (mode 1), per-token fp8 (mode 2), per-128-group (mode 3) and MX E5M2 and E2M1
    (modes 4/5) rows, element by element from exact rational arithmetic rounded once per
    binary32 operation, plus closed-form examples and invariants (group boundaries, all-zero
    groups, the ragged last group, the nibble order of packed E2M1 codes);
  * E2M1 encoding against a nearest-value search over the eight OCP fp4 magnitudes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle
import workloads
from exact import f32_bits, round_half_even, to_f32

E4M3, E5M2, E2M1 = oracle.CODE_E4M3, oracle.CODE_E5M2, oracle.CODE_E2M1
FP8_KIND = {E4M3: "e4m3", E5M2: "e5m2"}
FP8_MAX = {E4M3: 448, E5M2: 57344}
FP8_MAX_CODE = {E4M3: 0x7E, E5M2: 0x7B}


def bf16(vals):
    return workloads.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _row(rng, H, spread=(1e-3, 1.0, 50.0)):
    xf = (rng.standard_normal(H) * rng.choice(spread, H)).astype(np.float32)
    xb = workloads.f32_to_bf16_bits(xf)
    return xb, workloads.bf16_bits_to_f32(xb)


# ---------------------------------------------------------------------------------------
# E5M2
# ---------------------------------------------------------------------------------------

def test_e5m2_decode_matches_ieee_half():
    for code in range(256):
        want = np.array([code << 8], np.uint16).view(np.float16)[0]
        got = oracle.e5m2_to_f32(code)
        if np.isnan(want):
            assert math.isnan(got), hex(code)
        else:
            assert got == float(want), hex(code)
    assert oracle.e5m2_to_f32(0x7B) == 57344.0 and math.isinf(oracle.e5m2_to_f32(0x7C))


def test_e5m2_decode_table():
    for code, v in brute.e5m2_values():
        assert Fraction(oracle.e5m2_to_f32(code)) == v
        assert Fraction(oracle.e5m2_to_f32(code | 0x80)) == -v


def test_e5m2_all_bf16_inputs():
    """All finite bf16 values against the nearest-value search, with saturation."""
    mags = brute.e5m2_values()
    vals_f = np.array([float(v) for _, v in mags])
    codes = np.array([c for c, _ in mags])
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(b)
    fin = np.isfinite(f)
    for bits, v in zip(b[fin], f[fin]):
        a = abs(float(v))
        if a >= 57344:
            want = 0x7B
        else:
            d = np.abs(vals_f - a)
            best = np.flatnonzero(d == d.min())
            want = int(codes[best[0]] if len(best) == 1 else codes[best][codes[best] % 2 == 0][0])
        want |= 0x80 if (int(bits) & 0x8000) else 0
        assert oracle.e5m2_from_f32(float(v)) == want, hex(int(bits))


def test_e5m2_midpoints_against_nearest_search():
    mags = [v for _, v in brute.e5m2_values()]
    probes = set()
    for a, b in zip(mags, mags[1:]):
        mid = float((a + b) / 2)
        probes.update([mid, np.nextafter(np.float32(mid), np.float32(0)).item(),
                       np.nextafter(np.float32(mid), np.float32(1e9)).item()])
    probes.update([57344.0, 61439.0, 61440.0, 1e30, 2.0 ** -17, 2.0 ** -16, 3 * 2.0 ** -17])
    for v in sorted(probes):
        f = float(np.float32(v))
        for sv in (f, -f):
            assert oracle.e5m2_from_f32(sv) == brute.e5m2_nearest(Fraction(sv)), sv


def test_e5m2_matches_torch_in_range():
    import torch
    rng = np.random.default_rng(17)
    v = (rng.standard_normal(20000) * rng.choice([1e-6, 1e-3, 1, 1e3, 1e4], 20000)
         ).astype(np.float32)
    v = v[np.abs(v) < 57344]
    want = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([oracle.e5m2_from_f32(float(a)) for a in v], np.uint8)
    assert (got == want).all()


# ---------------------------------------------------------------------------------------
# int8 cast, E8M0, code types, scale counts
# ---------------------------------------------------------------------------------------

def test_int8_cast_ties_and_saturation():
    cases = {0.5: 0, 1.5: 2, 2.5: 2, -2.5: -2, -3.5: -4, 126.5: 126, 127.49: 127,
             127.5: 127, 200.0: 127, -127.5: -127, -1e30: -127, math.inf: 127,
             -math.inf: -127, math.nan: 0, -0.4: 0}
    for v, want in cases.items():
        assert oracle.int8_from_f32(v) == want, v


def test_e8m0_of_every_mx_scale():
    for e in range(-127, 128):
        s = np.float32(math.ldexp(1.0, e))
        assert float(s) == math.ldexp(1.0, e)             # exact, 2^-127 as a subnormal
        assert oracle.e8m0_from_scale(float(s)) == e + 127


def test_code_types_follow_the_mode_constraints():
    # default element type of each mode, then which explicit types each mode accepts
    assert [oracle.code_type(m) for m in range(6)] == [0, 1, 1, 2, 2, 2]
    allowed = {0: [], 1: [1], 2: [1, 2, 3], 3: [2, 3], 4: [2, 3, 4], 5: [2, 3, 4]}
    for m in range(6):
        for t in (1, 2, 3, 4, 5):
            assert (oracle.code_type(m, t) == t) == (t in allowed[m]), (m, t)
    assert oracle.code_type(6) == -1


def test_scale_counts():
    assert [oracle.scale_count(m, 7168) for m in range(6)] == [0, 0, 1, 56, 224, 224]
    assert oracle.scale_count(3, 1030) == 9 and oracle.scale_count(3, 1024) == 8
    assert oracle.scale_count(4, 1030) == 34 and oracle.scale_count(5, 1056) == 34


# ---------------------------------------------------------------------------------------
# mode 1: static int8
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("pre_kind", ["scalar", "row"])
def test_static_int8_exact(pre_kind):
    rng = np.random.default_rng(31)
    H = 300
    xb, xf = _row(rng, H, (1.0, 3.0))
    pre = (rng.uniform(16, 48, 1) if pre_kind == "scalar" else
           rng.uniform(16, 48, H)).astype(np.float32)
    q, sc = oracle.quant_row(1, xb, pre)
    assert len(sc) == 0
    saturated = 0
    for h in range(H):
        p = float(pre[0] if pre_kind == "scalar" else pre[h])
        prod = to_f32(Fraction(float(xf[h])) * Fraction(p))
        want = max(-127, min(127, round_half_even(Fraction(prod))))
        saturated += abs(round_half_even(Fraction(prod))) > 127
        assert q[h] == want, h
    assert saturated > 0                                # the clamp is exercised


def test_static_int8_closed_form():
    x = bf16([1.0, -1.5, 0.25, 3.0, -4.0, 0.0])
    q, _ = oracle.quant_row(1, x, np.array([42.0], np.float32))
    # 42, -63, 10.5 -> 10 (tie to even), 126, -168 -> -127, 0
    assert q.tolist() == [42, -63, 10, 126, -127, 0]


# ---------------------------------------------------------------------------------------
# dynamic fp8: mode 2 (whole row) and mode 3 (groups of 128)
# ---------------------------------------------------------------------------------------

def _dynamic_segment_check(ct, f, q, scale):
    """One dynamic segment: dyn = max / amax, codes = fp8(f * dyn), scale = 1 / dyn, each
    binary32 operation rounded once; NaN products (all-zero segment) encode as 0."""
    amax = float(np.max(np.abs(f)))
    if amax == 0.0:
        assert (q == 0).all() and scale == 0.0
        return
    dyn = to_f32(Fraction(FP8_MAX[ct]) / Fraction(amax)) if ct != oracle.CODE_INT8 else \
        to_f32(Fraction(127) / Fraction(amax))
    for fv, qv in zip(f, q):
        prod = to_f32(Fraction(float(fv)) * Fraction(dyn))
        if ct == oracle.CODE_INT8:
            want = max(-127, min(127, round_half_even(Fraction(prod))))
        else:
            want = brute.fp8_nearest(FP8_KIND[ct], Fraction(prod))
            if prod == 0.0:
                want = 0x80 if math.copysign(1, prod) < 0 else 0
        assert int(qv) == want, (float(fv), prod)
    assert f32_bits(scale) == f32_bits(to_f32(Fraction(1) / Fraction(dyn)))
    # the largest element reaches the type's largest code
    top = int(np.argmax(np.abs(f)))
    if ct != oracle.CODE_INT8:
        assert int(q[top]) & 0x7F == FP8_MAX_CODE[ct]


@pytest.mark.parametrize("ct", [E4M3, E5M2])
@pytest.mark.parametrize("pre_kind", [None, "scalar", "row"])
def test_per_token_fp8_exact(ct, pre_kind):
    rng = np.random.default_rng(41 + ct)
    for H in (64, 257):
        xb, xf = _row(rng, H)
        pre = None if pre_kind is None else (
            rng.uniform(0.5, 1.5, 1 if pre_kind == "scalar" else H).astype(np.float32))
        q, sc = oracle.quant_row(2, xb, pre, ct)
        assert len(sc) == 1
        f = xf if pre is None else np.array(
            [to_f32(Fraction(float(a)) * Fraction(float(pre[0] if len(pre) == 1 else pre[h])))
             for h, a in enumerate(xf)], np.float32)
        _dynamic_segment_check(ct, f, q.view(np.uint8), float(sc[0]))


@pytest.mark.parametrize("ct", [E4M3, E5M2])
def test_per_group_exact_with_ragged_tail(ct):
    rng = np.random.default_rng(51 + ct)
    H = 1030                                            # 8 full groups and one of 6
    xb, xf = _row(rng, H)
    xf_groups = [xf[g * 128:(g + 1) * 128] for g in range(9)]
    q, sc = oracle.quant_row(3, xb, None, ct)
    assert len(sc) == 9
    for g in range(9):
        _dynamic_segment_check(ct, xf_groups[g], q[g * 128:(g + 1) * 128], float(sc[g]))


@pytest.mark.parametrize("ct", [E4M3, E5M2])
def test_per_group_boundaries_and_zero_group(ct):
    # group g holds the value 2^g at its first element and 2^(g-1) elsewhere, except group 3,
    # which is all zero: each group's scale is 2^g / fp8_max, so one misplaced boundary or a
    # whole-row maximum shows at once
    H = 1024
    vals = np.zeros(H, np.float32)
    for g in range(8):
        if g == 3:
            continue
        vals[g * 128:(g + 1) * 128] = 2.0 ** (g - 1)
        vals[g * 128] = 2.0 ** g
    q, sc = oracle.quant_row(3, bf16(vals), None, ct)
    for g in range(8):
        blk = q[g * 128:(g + 1) * 128]
        if g == 3:
            assert sc[g] == 0.0 and (blk == 0).all()
            continue
        assert sc[g] == np.float32(1) / (np.float32(FP8_MAX[ct]) / np.float32(2.0 ** g))
        assert blk[0] == FP8_MAX_CODE[ct]
        half = brute.fp8_nearest(FP8_KIND[ct], Fraction(FP8_MAX[ct], 2))
        assert (blk[1:] == half).all()


# ---------------------------------------------------------------------------------------
# MX with E5M2 elements
# ---------------------------------------------------------------------------------------

def test_mx_e5m2_closed_forms():
    codes, sc = oracle.quant_row(4, bf16([1.0] * 32), None, E5M2)
    # floor(log2 1) - 15 = -15; 1 * 2^15 = 32768 = 1.0 * 2^15 -> exponent field 30 -> 0x78
    assert sc.tolist() == [2.0 ** -15, 0.0] and (codes == 0x78).all()
    codes, sc = oracle.quant_row(4, bf16([1.9] * 32), None, E5M2)
    # bf16(1.9) = 1.8984375; * 2^15 = 62208 > 57344 saturates
    assert sc[0] == 2.0 ** -15 and (codes == 0x7B).all()
    codes, sc = oracle.quant_row(4, bf16([3.0] + [0.0] * 30 + [-0.375]), None, E5M2)
    # amax 3 -> -14; 3 * 2^14 = 49152 = 1.5 * 2^15 -> 0x7A; 0.375 * 2^14 = 6144 = 1.5 * 2^12
    # -> exponent field 27, mantissa 2 -> 0x6E, negative 0xEE
    assert sc[0] == 2.0 ** -14 and codes[0] == 0x7A and codes[31] == 0xEE
    codes, sc = oracle.quant_row(5, np.zeros(32, np.uint16), None, E5M2)
    # 1e-4 / 57344 = 1.74e-9: log2 = -29.1 -> ceil -29
    assert sc[0] == 2.0 ** -29 and (codes == 0).all()
    codes, sc = oracle.quant_row(5, bf16([57344.0] * 32), None, E5M2)
    assert sc[0] == 1.0 and (codes == 0x7B).all()


@pytest.mark.parametrize("mode", [4, 5])
@pytest.mark.parametrize("ct", [E4M3, E5M2])
def test_mx_rows_exact_any_type(mode, ct):
    rng = np.random.default_rng(61 + mode + 2 * ct)
    emax = 8 if ct == E4M3 else 15
    for H in (1030, 1056):
        xf = (rng.standard_normal(H) * rng.choice([1e-30, 1e-6, 1.0, 300.0], H)).astype(np.float32)
        xb = workloads.f32_to_bf16_bits(xf)
        xf = workloads.bf16_bits_to_f32(xb)
        codes, sc = oracle.quant_row(mode, xb, None, ct)
        nb = (H + 31) // 32
        assert len(sc) == nb + (nb & 1) and (sc[nb:] == 0).all()
        for b in range(nb):
            blk = xf[b * 32:(b + 1) * 32]
            amax = Fraction(float(np.abs(blk).max()))
            if mode == 4:
                se = -127 if amax == 0 else max(-127, math.floor(math.log2(amax)) - emax)
                # exact floor(log2) for a power-of-two-adjacent amax
                if amax != 0 and se > -127:
                    while Fraction(2) ** (se + emax) > amax:
                        se -= 1
                    while Fraction(2) ** (se + emax + 1) <= amax:
                        se += 1
            else:
                c = to_f32(Fraction(max(amax, Fraction(float(np.float32(1e-4)))))
                           / Fraction(FP8_MAX[ct]))
                se = math.ceil(math.log2(c))
                while Fraction(2) ** se < Fraction(c):
                    se += 1
                while Fraction(2) ** (se - 1) >= Fraction(c):
                    se -= 1
            assert Fraction(float(sc[b])) == Fraction(2) ** se, (b, se)
            for v, code in zip(blk, codes[b * 32:(b + 1) * 32]):
                want = brute.fp8_nearest(FP8_KIND[ct], Fraction(float(v)) / Fraction(2) ** se)
                if v == 0:
                    want = 0x80 if math.copysign(1, float(v)) < 0 else 0
                assert code == want


def test_quant_row_rejects_mismatched_arguments():
    x = bf16([1.0] * 64)
    with pytest.raises(ValueError):
        oracle.quant_row(1, x)                          # static mode needs scales
    with pytest.raises(ValueError):
        oracle.quant_row(4, x, np.ones(64, np.float32))  # MX takes no scales
    with pytest.raises(ValueError):
        oracle.quant_row(2, x, np.ones(10, np.float32))  # neither scalar nor a row


# ---------------------------------------------------------------------------------------
# E2M1 (fp4) MX elements, two codes per byte
# ---------------------------------------------------------------------------------------

E2M1_VALUES = [0, 0.5, 1, 1.5, 2, 3, 4, 6]          # the OCP fp4 magnitudes, codes 0..7


def _e2m1_nearest(v):
    """Nearest E2M1 code to the exact value v (ties to the even code), |v| >= 6 -> 6."""
    sign = 0x8 if v < 0 else 0
    a = abs(Fraction(v))
    if a >= 6:
        return sign | 0x7
    best = min(range(8), key=lambda c: (abs(Fraction(E2M1_VALUES[c]) - a), c & 1))
    return sign | best


def test_e2m1_decode_table():
    for code, v in enumerate(E2M1_VALUES):
        assert oracle.e2m1_to_f32(code) == v
        assert oracle.e2m1_to_f32(code | 0x8) == -v


def test_e2m1_all_bf16_inputs():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(b)
    for v in f[np.isfinite(f)]:
        want = _e2m1_nearest(float(v))
        if v == 0:
            want = 0x8 if math.copysign(1, float(v)) < 0 else 0
        assert oracle.e2m1_from_f32(float(v)) == want, float(v)


def test_e2m1_ties():
    # midpoints go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2,
    # 2.5 -> 2, 3.5 -> 4, 5 -> 4; 6.5 and up saturate to 6
    for v, want in [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4),
                    (3.5, 0x6), (5.0, 0x6), (6.5, 0x7), (1e9, 0x7), (-5.0, 0xE)]:
        assert oracle.e2m1_from_f32(v) == want, v


def _unpack_e2m1(codes):
    out = np.empty(codes.size * 2, np.uint8)
    out[0::2] = codes & 0xF
    out[1::2] = codes >> 4
    return out


def test_mx_e2m1_closed_forms_and_packing():
    vals = [1.0] * 32
    vals[0], vals[1] = -1.5, 0.5
    codes, sc = oracle.quant_row(4, bf16(vals), None, E2M1)
    # amax 1.5 -> floor(log2) 0 - emax 2 = -2: elements times 4: -6 (0xF), 2 (0x4), 4 (0x6)
    assert len(codes) == 16 and sc.tolist() == [0.25, 0.0]
    assert codes[0] == (0xF | (0x4 << 4))           # element 0 in the low nibble
    assert (codes[1:] == (0x6 | (0x6 << 4))).all()
    codes, sc = oracle.quant_row(5, bf16([6.0] * 32), None, E2M1)
    assert sc[0] == 1.0 and (codes == 0x77).all()    # 6 / 6 = 1 -> exponent 0
    codes, sc = oracle.quant_row(5, np.zeros(32, np.uint16), None, E2M1)
    # 1e-4 / 6 = 1.67e-5: log2 = -15.87 -> ceil -15
    assert sc[0] == 2.0 ** -15 and (codes == 0).all()


@pytest.mark.parametrize("mode", [4, 5])
def test_mx_e2m1_rows_exact(mode):
    rng = np.random.default_rng(71 + mode)
    H = 1056
    xf = (rng.standard_normal(H) * rng.choice([1e-6, 1.0, 300.0], H)).astype(np.float32)
    xb = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xb)
    codes, sc = oracle.quant_row(mode, xb, None, E2M1)
    assert len(codes) == H // 2
    q = _unpack_e2m1(codes)
    for b in range((H + 31) // 32):
        blk = xf[b * 32:(b + 1) * 32]
        amax = Fraction(float(np.abs(blk).max()))
        if mode == 4:
            se = -127 if amax == 0 else max(-127, math.floor(math.log2(amax)) - 2)
            if amax != 0 and se > -127:
                while Fraction(2) ** (se + 2) > amax:
                    se -= 1
                while Fraction(2) ** (se + 3) <= amax:
                    se += 1
        else:
            c = to_f32(Fraction(max(amax, Fraction(float(np.float32(1e-4))))) / Fraction(6))
            se = math.ceil(math.log2(c))
            while Fraction(2) ** se < Fraction(c):
                se += 1
            while Fraction(2) ** (se - 1) >= Fraction(c):
                se -= 1
        assert Fraction(float(sc[b])) == Fraction(2) ** se
        for v, code in zip(blk, q[b * 32:(b + 1) * 32]):
            want = _e2m1_nearest(Fraction(float(v)) / Fraction(2) ** se)
            if v == 0:
                want = 0x8 if math.copysign(1, float(v)) < 0 else 0
            assert code == want


def test_e2m1_needs_even_hidden():
    with pytest.raises(ValueError):
        oracle.quant_row(4, bf16([1.0] * 33), None, E2M1)
