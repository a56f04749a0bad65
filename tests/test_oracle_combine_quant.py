"""Pins of the oracle's combine-side int8 block quantization (the SMP article's combine INT8
block quantization) against what the page and the number formats fix, independently of the
oracle's C code:

  * fp16 narrowing and widening against numpy's IEEE binary16 conversions;
  * the int8 cast of an fp16 value at its rounding ties and saturation points;
  * quantized rows element by element from exact rational arithmetic (amax * fp32(1/127),
    one correctly rounded division, numpy's float16 rounding, then round half to even),
    including a witness that the float -> fp16 -> int8 chain differs from one direct
    rounding; the 8-element block boundaries; all-zero blocks; the short last block;
  * the dequantization bound, and the int8 combine reducing to the pinned bf16 combine when
    every block's scale is exactly 1.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from exact import f32_bits, round_half_even, to_f32

INV127 = np.float32(1) / np.float32(127)


def bf16(vals):
    return workloads.f32_to_bf16_bits(np.asarray(vals, np.float32))


# ---------------------------------------------------------------------------------------
# fp16
# ---------------------------------------------------------------------------------------

def test_f16_decode_all_codes_against_numpy():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = codes.view(np.float16).astype(np.float32)
    for c, w in zip(codes[::7], want[::7]):
        got = oracle.f16_to_f32(int(c))
        assert (np.isnan(w) and np.isnan(got)) or got == w, hex(int(c))


def test_f16_encode_against_numpy():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # exact binary16 midpoints (13 dropped bits = 0x1000 pattern) in the normal range
    mids = (rng.integers(0x38800000, 0x477FE000, 3000, dtype=np.uint64).astype(np.uint32)
            & np.uint32(0xFFFFE000)) | np.uint32(0x1000)
    vals = np.concatenate([f, mids.view(np.float32), np.float32([65504, 65519.99, 65520,
                                                                 2.0 ** -24, 2.0 ** -25,
                                                                 3 * 2.0 ** -26, 0.0])])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(v)) for v in vals], np.uint16)
    assert (got == want).all()


def test_int8_from_f16_ties_and_saturation():
    cases = {2.5: 2, 3.5: 4, -2.5: -2, 0.5: 0, 126.5: 126, 127.5: 127, 200.0: 127,
             -65504.0: -127, 1.5: 2}
    for v, want in cases.items():
        h = int(np.float16(v).view(np.uint16))
        assert oracle.int8_from_f16(h) == want, v
    assert oracle.int8_from_f16(0x7E00) == 0                     # NaN


# ---------------------------------------------------------------------------------------
# block quantization
# ---------------------------------------------------------------------------------------

def _expected_block(xf):
    """(codes, scale) of one block from exact arithmetic and numpy's float16 rounding."""
    amax = float(np.max(np.abs(xf)))
    scale = to_f32(Fraction(amax) * Fraction(float(INV127)))
    if scale == 0.0:
        return [0] * len(xf), 0.0
    out = []
    for v in xf:
        q = to_f32(Fraction(float(v)) / Fraction(scale))
        h = float(np.float16(q))                    # IEEE round to nearest even
        out.append(max(-127, min(127, round_half_even(Fraction(h)))))
    return out, scale


@pytest.mark.parametrize("H", [1024, 1030, 4100])
def test_quant_rows_exact(H):
    rng = np.random.default_rng(H)
    xf = (rng.standard_normal(H) * rng.choice([1e-30, 1e-3, 1.0, 300.0], H)).astype(np.float32)
    xf[16:24] = 0.0                                 # one all-zero block
    xb = workloads.f32_to_bf16_bits(xf)
    xf = workloads.bf16_bits_to_f32(xb)
    q, sc = oracle.combine_quant_row(xb)
    nb = (H + 7) // 8
    assert len(sc) == nb
    for b in range(nb):
        blk = xf[b * 8:(b + 1) * 8]
        codes, scale = _expected_block(blk)
        assert f32_bits(float(sc[b])) == f32_bits(scale), b
        assert q[b * 8:(b + 1) * 8].tolist() == codes, b
    assert sc[2] == 0.0 and (q[16:24] == 0).all()


def test_double_rounding_chain_is_followed():
    """Find elements whose quotient x/scale lies within an fp16 step of a .5 tie: there the
    float -> fp16 -> int8 chain and a single rounding can differ, and the oracle must give
    the chain's answer."""
    rng = np.random.default_rng(9)
    witnesses = 0
    for _ in range(400):
        xb = workloads.f32_to_bf16_bits(rng.standard_normal(8).astype(np.float32))
        xf = workloads.bf16_bits_to_f32(xb)
        q, sc = oracle.combine_quant_row(xb)
        for v, code in zip(xf, q):
            qf = to_f32(Fraction(float(v)) / Fraction(float(sc[0])))
            chain = max(-127, min(127, round_half_even(Fraction(float(np.float16(qf))))))
            direct = max(-127, min(127, round_half_even(Fraction(qf))))
            assert code == chain
            witnesses += chain != direct
    assert witnesses > 0


def test_block_boundaries_and_short_last_block():
    # block b holds 2^b at its last element and 1.0 elsewhere; H = 20 -> blocks of 8, 8, 4
    vals = np.ones(20, np.float32)
    vals[7], vals[15], vals[19] = 1.0, 2.0, 4.0
    q, sc = oracle.combine_quant_row(bf16(vals))
    assert [float(v) for v in sc] == [float(np.float32(a) * INV127) for a in (1.0, 2.0, 4.0)]
    assert (q[:8] == 127).all()                     # amax 1: every element is the maximum
    assert q[15] == 127 and q[19] == 127
    assert (q[8:15] == round_half_even(Fraction(127, 2))).all()   # 63.5 -> 64
    assert (q[16:19] == round_half_even(Fraction(127, 4))).all()  # 31.75 -> 32


def test_integer_rows_with_127_have_unit_scale():
    rng = np.random.default_rng(1)
    x = rng.integers(-127, 128, 64).astype(np.float32)
    x[::8] = 127.0
    q, sc = oracle.combine_quant_row(bf16(x))
    assert (sc == 1.0).all() and (q == x.astype(np.int8)).all()


def test_dequant_exact_and_error_bound():
    rng = np.random.default_rng(2)
    q = rng.integers(-127, 128, 40).astype(np.int8)
    sc = rng.uniform(1e-3, 10, 5).astype(np.float32)
    out = oracle.combine_dequant_row(q, sc)
    for h in range(40):
        assert f32_bits(float(out[h])) == f32_bits(to_f32(Fraction(int(q[h])) *
                                                          Fraction(float(sc[h // 8]))))
    xb = workloads.f32_to_bf16_bits(rng.standard_normal(1024).astype(np.float32) * 5)
    xf = workloads.bf16_bits_to_f32(xb).astype(np.float64)
    q, sc = oracle.combine_quant_row(xb)
    deq = oracle.combine_dequant_row(q, sc).astype(np.float64)
    step = np.repeat(sc.astype(np.float64), 8)
    assert (np.abs(deq - xf) <= (0.5 + 2.0 ** -5) * step + np.abs(xf) * 2.0 ** -20).all()


# ---------------------------------------------------------------------------------------
# whole-buffer quantize and the int8 combine
# ---------------------------------------------------------------------------------------

def _dispatch_tiny(seed, **kw):
    wl = workloads.C1_MODE0.replace(**kw)
    inp = workloads.generate(wl, seed=seed)
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, zero_expert_num=wl.zero_expert_num,
                          copy_expert_num=wl.copy_expert_num, mask_kind=wl.mask_kind)
    d = oracle.dispatch(cfg, inp["x"], inp["expert_ids"], mask=inp.get("mask"))
    return wl, cfg, inp, d


def test_quantize_touches_only_routed_rows():
    wl, cfg, inp, d = _dispatch_tiny(1, mask_kind=2, inactive_tokens_per_rank=4)
    P = int(d["recv_offsets"][-1])
    assert P < wl.cap
    eo = workloads.f32_to_bf16_bits(np.random.default_rng(0).standard_normal(
        (wl.cap, wl.H)).astype(np.float32))
    codes, scales = oracle.combine_quantize(cfg, eo, d["recv_offsets"])
    for r in (0, P // 2, P - 1):
        q, sc = oracle.combine_quant_row(eo[r])
        assert (codes[r] == q).all() and (scales[r] == sc).all()
    assert (codes[P:] == 0).all() and (scales[P:] == 0).all()


def test_int8_combine_reduces_to_the_bf16_combine_at_unit_scales():
    """Integer expert rows with a 127 in every block quantize with scale 1 and codes equal to
    the values; the int8 combine must then equal the (separately pinned) bf16 combine."""
    wl, cfg, inp, d = _dispatch_tiny(2, zero_expert_num=1, copy_expert_num=1, mask_kind=2,
                                     inactive_tokens_per_rank=3, routing="randint")
    rng = np.random.default_rng(4)
    vals = rng.integers(-127, 128, (wl.cap, wl.H)).astype(np.float32)
    vals[:, ::8] = 127.0
    eo = workloads.f32_to_bf16_bits(vals)
    codes, scales = oracle.combine_quantize(cfg, eo, d["recv_offsets"])
    P = int(d["recv_offsets"][-1])
    assert (scales[:P] == 1.0).all()
    args = (inp["expert_ids"], d["expand_idx"], inp["expert_scales"], d["ep_recv_count"],
            d["recv_offsets"])
    y8 = oracle.combine_int8(cfg, codes, scales, *args, mask=inp["mask"], ori_x=inp["x"])
    y16 = oracle.combine(cfg, eo, *args, mask=inp["mask"], ori_x=inp["x"])
    assert (y8 == y16).all()


def test_int8_combine_close_to_the_bf16_combine():
    """On N(0,1) expert rows the int8 round trip changes y by at most the quantization
    error: per pick half a step (plus the fp16 step) times the weight."""
    wl, cfg, inp, d = _dispatch_tiny(3)
    eo = workloads.f32_to_bf16_bits(np.random.default_rng(5).standard_normal(
        (wl.cap, wl.H)).astype(np.float32))
    codes, scales = oracle.combine_quantize(cfg, eo, d["recv_offsets"])
    args = (inp["expert_ids"], d["expand_idx"], inp["expert_scales"], d["ep_recv_count"],
            d["recv_offsets"])
    y8 = workloads.bf16_bits_to_f32(oracle.combine_int8(cfg, codes, scales, *args))
    y16 = workloads.bf16_bits_to_f32(oracle.combine(cfg, eo, *args))
    bound = np.zeros((wl.W, wl.BS, wl.H))
    for s in range(wl.W):
        for i in range(wl.BS):
            for k in range(wl.K):
                e = inp["expert_ids"][s, i, k]
                row = oracle.dest_row(cfg, d["ep_recv_count"], d["recv_offsets"], s, e,
                                      d["expand_idx"][s, i, k])
                step = np.repeat(scales[row].astype(np.float64), 8)[:wl.H]
                bound[s, i] += abs(float(inp["expert_scales"][s, i, k])) * (0.5 + 2.0 ** -5) * step
    bf16_ulp = 2.0 ** -7 * np.maximum(np.abs(y16), np.abs(y8))
    assert (np.abs(y8 - y16) <= bound + 2 * bf16_ulp + 1e-30).all()


def test_token_version_equals_the_whole_buffer_version():
    wl, cfg, inp, d = _dispatch_tiny(6, zero_expert_num=1, copy_expert_num=1, mask_kind=2,
                                     inactive_tokens_per_rank=2, routing="randint")
    eo = workloads.f32_to_bf16_bits(np.random.default_rng(8).standard_normal(
        (wl.cap, wl.H)).astype(np.float32))
    codes, scales = oracle.combine_quantize(cfg, eo, d["recv_offsets"])
    args = (inp["expert_ids"], d["expand_idx"], inp["expert_scales"], d["ep_recv_count"],
            d["recv_offsets"])
    y = oracle.combine_int8(cfg, codes, scales, *args, mask=inp["mask"], ori_x=inp["x"])
    for s in range(wl.W):
        for i in range(wl.BS):
            yt = oracle.combine_int8_token(cfg, codes, scales, *args, s, i, mask=inp["mask"],
                                           ori_x=inp["x"])
            assert (yt == y[s, i]).all()
