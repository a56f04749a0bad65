"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test ties an oracle function to something other than itself: the page's printed
worked example, a brute-force enumeration, exact rational arithmetic, closed forms, library
routines on special cases, or invariants the pages imply.  A plausible slip in the oracle
(a dropped term, a wrong index or sign, a transposed matrix, a different operation order or
rounding) fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle
import workloads
from exact import f32_bits, round_half_even, to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16(vals):
    return workloads.f32_to_bf16_bits(np.asarray(vals, np.float32))


# ---------------------------------------------------------------------------------------
# routing: the page's worked example
# ---------------------------------------------------------------------------------------

def _ids_for_receiver0(M, W, L, BS):
    """K=1 routing in which source s sends M[e][s] tokens to expert e (e < L, receiver 0)
    and every other token to receiver 1's first expert."""
    ids = np.full((W, BS, 1), L, np.int32)  # expert L lives on rank 1
    for s in range(W):
        t = 0
        for e in range(L):
            for _ in range(M[e][s]):
                ids[s, t, 0] = e
                t += 1
    return ids


def test_worked_example_sendcounts():
    g = json.load(open(os.path.join(GOLDEN, "ddd_sendcounts_example.json")))
    W, L = g["W"], g["L"]
    pref = g["send_counts_prefix"]
    flat = [v for row in pref for v in row]
    # per-(expert, rank) counts implied by the printed running totals
    M = [[flat[e * W + s] - (flat[e * W + s - 1] if e * W + s > 0 else 0)
          for s in range(W)] for e in range(L)]
    assert M == [[1, 0, 1, 1], [0, 5, 2, 2]]
    BS = 8
    ids = _ids_for_receiver0(M, W, L, BS)
    for typ in (0, 1):
        cfg = oracle.make_cfg(W, W * L, BS, 1024, 1, expert_token_nums_type=typ)
        cnt, eidx = oracle.route(cfg, ids)
        erc, etn, off = oracle.recv_counts(cfg, cnt)
        assert erc[0].tolist() == flat
        # expert_token_nums is the last column of the matrix (type 0) or plain counts
        want = [pref[e][-1] for e in range(L)] if typ == 0 else [sum(M[e]) for e in range(L)]
        assert etn[0].tolist() == want
        assert off[0] == 0 and off[1] == flat[-1]
        for wk in g["worked"]:
            e, r = wk["expert"], wk["rank"]
            start = int(oracle.dest_row(cfg, erc, off, r, e, 0))
            assert start == wk["start"]
            assert M[e][r] == wk["count"]


# ---------------------------------------------------------------------------------------
# routing: brute force on tiny inputs
# ---------------------------------------------------------------------------------------

def _check_route_against_brute(W, E, BS, K, ids, mask, mask_kind, Z=0, C=0):
    for typ in (0, 1):
        cfg = oracle.make_cfg(W, E, BS, 1024, K, zero_expert_num=Z, copy_expert_num=C,
                              expert_token_nums_type=typ, mask_kind=mask_kind)
        cnt, eidx = oracle.route(cfg, ids, mask)
        erc, etn, off = oracle.recv_counts(cfg, cnt)
        rows, beidx, berc, bcnt, bcum, boff = brute.route(W, E, BS, K, ids.tolist(),
                                                          None if mask is None else mask.tolist(),
                                                          mask_kind)
        assert eidx.tolist() == beidx
        assert erc.tolist() == berc
        assert etn.tolist() == (bcum if typ == 0 else bcnt)
        assert off.tolist() == boff
        for (s, i, k), row in rows.items():
            assert oracle.dest_row(cfg, erc, off, s, int(ids[s, i, k]), int(eidx[s, i, k])) == row


def test_route_exhaustive_micro():
    """Every routing of 2 ranks x 2 tokens with 2 distinct picks among 4 experts."""
    W, E, BS, K = 2, 4, 2, 2
    picks = list(itertools.permutations(range(E), K))       # 12 ordered distinct pairs
    cfg = oracle.make_cfg(W, E, BS, 1024, K)
    n = 0
    for combo in itertools.product(picks, repeat=W * BS):
        ids = np.array(combo, np.int32).reshape(W, BS, K)
        cnt, eidx = oracle.route(cfg, ids)
        erc, etn, off = oracle.recv_counts(cfg, cnt)
        rows, beidx, berc, bcnt, _, boff = brute.route(W, E, BS, K, ids.tolist())
        assert eidx.tolist() == beidx
        assert erc.tolist() == berc
        assert off.tolist() == boff
        n += 1
    assert n == 12 ** 4


@pytest.mark.parametrize("seed", range(40))
def test_route_random_tiny(seed):
    rng = np.random.default_rng(1000 + seed)
    W = int(rng.integers(2, 5))
    L = int(rng.integers(1, 4))
    E = W * L
    BS = int(rng.integers(1, 7))
    K = int(rng.integers(1, 5))
    Z = int(rng.integers(0, 3))
    C = int(rng.integers(0, 3))
    ids = rng.integers(0, E + Z + C, size=(W, BS, K)).astype(np.int32)   # duplicates allowed
    mask_kind = int(rng.integers(0, 3))
    if mask_kind == 0:
        mask = None
    elif mask_kind == 1:
        mask = np.zeros((W, BS), np.uint8)
        for s in range(W):
            mask[s, :int(rng.integers(0, BS + 1))] = 1
    else:
        mask = (rng.random((W, BS, K)) < 0.7).astype(np.uint8)
    _check_route_against_brute(W, E, BS, K, ids, mask, mask_kind, Z, C)


def test_route_rejects_out_of_range_ids():
    cfg = oracle.make_cfg(2, 4, 1, 1024, 1, zero_expert_num=1)
    with pytest.raises(ValueError):
        oracle.route(cfg, np.array([[[5]], [[0]]], np.int32))
    with pytest.raises(ValueError):
        oracle.route(cfg, np.array([[[-1]], [[0]]], np.int32))


def test_route_invariants_c2_shape():
    wl = workloads.C2
    inp = workloads.generate(wl, seed=0)
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K)
    cnt, eidx = oracle.route(cfg, inp["expert_ids"])
    erc, etn, off = oracle.recv_counts(cfg, cnt)
    ids = inp["expert_ids"]
    # sum of per-expert token counts = routed picks (all picks are routed here)
    assert etn.sum() == wl.W * wl.BS * wl.K == off[-1]
    # per (source, expert) the ordinals are 0..M-1 in token order
    for s in range(wl.W):
        for e in range(wl.E):
            sel = eidx[s][ids[s] == e]
            assert sel.tolist() == list(range(cnt[s, e]))
    # every receiver's rows form a permutation of its window
    L = wl.L
    rows = np.array([oracle.dest_row(cfg, erc, off, s, int(ids[s, i, k]), int(eidx[s, i, k]))
                     for s in range(wl.W) for i in range(wl.BS) for k in range(wl.K)])
    assert sorted(rows.tolist()) == list(range(off[-1]))
    # type 0 is the running sum of type 1 and equals the last column of ep_recv_count
    cfg0 = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, expert_token_nums_type=0)
    _, etn0, _ = oracle.recv_counts(cfg0, cnt)
    assert (etn0 == np.cumsum(etn, axis=1)).all()
    assert (etn0 == erc.reshape(wl.W, L, wl.W)[:, :, -1]).all()


# ---------------------------------------------------------------------------------------
# bf16 and E4M3 conversions
# ---------------------------------------------------------------------------------------

def test_bf16_roundtrip_and_rounding_against_torch():
    import torch
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # add exact halfway patterns (low 16 bits = 0x8000) with odd and even kept halves
    u[:2000] = (u[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(v) for v in f], np.uint16)
    assert (got == want).all()
    for b in (0x0001, 0x3F80, 0xBF80, 0x7F7F, 0x8000, 0x0080):
        assert f32_bits(oracle.bf16_to_f32(b)) == b << 16


def test_e4m3_decode_table():
    for code, v in brute.e4m3_values():
        assert Fraction(oracle.e4m3_to_f32(code)) == v
        assert Fraction(oracle.e4m3_to_f32(code | 0x80)) == -v
    assert oracle.e4m3_to_f32(0x7E) == 448.0
    assert math.isnan(oracle.e4m3_to_f32(0x7F))


def _e4m3_probe_values():
    vals = set()
    # every value with an 8-bit significand across the binades that reach E4M3
    for ex in range(-20, 12):
        for m in range(128, 256):
            vals.add(m * 2.0 ** (ex - 7))
    # exact midpoints between neighbouring E4M3 values, and their float neighbours
    mags = [v for _, v in brute.e4m3_values()]
    for a, b in zip(mags, mags[1:]):
        mid = float((a + b) / 2)
        vals.update([mid, np.nextafter(np.float32(mid), np.float32(0)).item(),
                     np.nextafter(np.float32(mid), np.float32(1e9)).item()])
    vals.update([448.0, 464.0, 480.0, 1e6, 2.0 ** -10, 2.0 ** -9, 2.0 ** -11, 0.0])
    return sorted(vals)


def test_e4m3_rounding_against_nearest_search():
    for v in _e4m3_probe_values():
        f = float(np.float32(v))
        for sv in (f, -f):
            want = brute.e4m3_nearest(Fraction(sv))
            if sv == 0.0 and math.copysign(1, sv) < 0:
                want = 0x80
            assert oracle.e4m3_from_f32(sv) == want, (sv, hex(want))


def test_e4m3_all_bf16_inputs():
    """All 65,280 finite bf16 values, compared with the nearest-value search."""
    mags = brute.e4m3_values()
    vals_f = np.array([float(v) for _, v in mags])
    codes = np.array([c for c, _ in mags])
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(b)
    fin = np.isfinite(f)
    for bits, v in zip(b[fin], f[fin]):
        a = abs(float(v))
        if a >= 448:
            want = 0x7E
        else:
            d = np.abs(vals_f - a)
            best = np.flatnonzero(d == d.min())
            want = int(codes[best[0]] if len(best) == 1 else codes[best][codes[best] % 2 == 0][0])
        want |= 0x80 if (int(bits) & 0x8000) else 0
        assert oracle.e4m3_from_f32(float(v)) == want, hex(int(bits))


# ---------------------------------------------------------------------------------------
# int8 per-token quantization (quant_mode 2)
# ---------------------------------------------------------------------------------------

def test_int8_closed_form_example():
    # amax 2 -> dyn = 127/2 = 63.5 exactly; products 63.5, -127, 31.75, 47.625 round half
    # to even: 64, -127, 32, 48; scale = fp32(1/63.5) = fp32(2/127)
    x = bf16([1.0, -2.0, 0.5, 0.75])
    q, sc = oracle.quant_int8_row(x)
    assert q.tolist() == [64, -127, 32, 48]
    assert f32_bits(sc) == f32_bits(to_f32(Fraction(2, 127)))


def test_int8_all_zero_row():
    q, sc = oracle.quant_int8_row(np.zeros(64, np.uint16))
    assert (q == 0).all() and sc == 0.0


def _int8_exact_check(xf, smooth, q, sc):
    f = xf if smooth is None else np.array([to_f32(Fraction(float(a)) * Fraction(float(b)))
                                            for a, b in zip(xf, smooth)], np.float32)
    amax = float(np.max(np.abs(f)))
    dyn = to_f32(Fraction(127) / Fraction(amax))
    for fv, qv in zip(f, q):
        prod = to_f32(Fraction(float(fv)) * Fraction(dyn))
        assert qv == max(-127, min(127, round_half_even(Fraction(prod))))
    assert f32_bits(sc) == f32_bits(to_f32(Fraction(1) / Fraction(dyn)))
    # invariants: |q| <= 127 with 127 reached at the absolute maximum; dequant error is at
    # most half a step plus binary32 slack
    assert np.abs(q.astype(np.int32)).max() == 127
    assert np.abs(q.astype(np.int32)[np.argmax(np.abs(f))]) == 127
    err = np.abs(q.astype(np.float64) * sc - f.astype(np.float64))
    assert (err <= 0.5 * sc + np.abs(f) * 2.0 ** -20 + 1e-30).all()


@pytest.mark.parametrize("smoothed", [False, True])
def test_int8_rows_exact(smoothed):
    rng = np.random.default_rng(11 + smoothed)
    for _ in range(6):
        H = int(rng.integers(16, 200))
        xf = rng.standard_normal(H).astype(np.float32) * np.float32(rng.choice([1e-3, 1, 50]))
        xf[rng.random(H) < 0.05] *= 10
        xb = workloads.f32_to_bf16_bits(xf)
        xf = workloads.bf16_bits_to_f32(xb)
        sm = rng.uniform(0.5, 1.5, H).astype(np.float32) if smoothed else None
        q, sc = oracle.quant_int8_row(xb, sm)
        _int8_exact_check(xf, sm, q, sc)


def test_int8_scale_all_bf16_amax():
    """dyn = 127/amax and scale = 1/dyn correctly rounded, for every positive finite bf16
    amax (checked through a one-element row, whose code must be 127)."""
    for b in range(0x0001, 0x7F80):
        amax = oracle.bf16_to_f32(b)
        q, sc = oracle.quant_int8_row(np.array([b], np.uint16))
        dyn = to_f32(Fraction(127) / Fraction(amax))
        want = 0.0 if math.isinf(dyn) else to_f32(Fraction(1) / Fraction(dyn))
        assert f32_bits(sc) == f32_bits(want), hex(b)
        assert q[0] == 127


def test_int8_matches_numpy_float32_without_smooth():
    """Library special case: without smooth scales the whole mode is numpy float32
    division, multiply and rint."""
    rng = np.random.default_rng(3)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal(7168).astype(np.float32))
    xf = workloads.bf16_bits_to_f32(xb)
    q, sc = oracle.quant_int8_row(xb)
    dyn = np.float32(127) / np.max(np.abs(xf))
    assert (q == np.rint(xf * dyn).astype(np.int8)).all()
    assert sc == np.float32(1) / dyn


# ---------------------------------------------------------------------------------------
# MX quantization (quant_modes 4 and 5)
# ---------------------------------------------------------------------------------------

def test_mx_closed_form_examples():
    ones = bf16([1.0] * 32)
    codes, sc = oracle.quant_mx_row(ones, clip=False)
    # floor(log2 1) - 8 = -8: 1 / 2^-8 = 256 = 1.0 * 2^8 -> exponent field 15, mantissa 0
    assert sc.tolist() == [2.0 ** -8, 0.0] and (codes == 0x78).all()
    blk = bf16([3.0] + [0.0] * 30 + [-1.875])
    codes, sc = oracle.quant_mx_row(blk, clip=False)
    # amax 3 -> shared exp -7; 3 * 128 = 384 = 1.5 * 2^8 -> 0x7C; 1.875*128 = 240 = 1.875*2^7
    # -> exponent field 14, mantissa 7 -> 0x77 (negative: 0xF7)
    assert sc[0] == 2.0 ** -7 and codes[0] == 0x7C and codes[31] == 0x80 | 0x77
    codes, sc = oracle.quant_mx_row(bf16([1.875] * 32), clip=False)
    # 1.875 * 256 = 480 > 448 saturates
    assert sc[0] == 2.0 ** -8 and (codes == 0x7E).all()
    # clip variant
    codes, sc = oracle.quant_mx_row(np.zeros(32, np.uint16), clip=True)
    # max(0, 1e-4)/448 = 2.23e-7; log2 = -13.29 - 8.81 = -22.1 -> ceil = -22
    assert sc[0] == 2.0 ** -22 and (codes == 0).all()
    codes, sc = oracle.quant_mx_row(bf16([448.0] * 32), clip=True)
    assert sc[0] == 1.0 and (codes == 0x7E).all()
    codes, sc = oracle.quant_mx_row(bf16([896.0, 449.0] + [0.0] * 30), clip=True)
    # 896/448 = 2 -> exp 1: 896/2 = 448 (0x7E); bf16(449) = 448, so 448/2 = 224 (0x76)
    assert sc[0] == 2.0 and codes[0] == 0x7E and codes[1] == 0x76


@pytest.mark.parametrize("clip", [False, True])
def test_mx_rows_invariants(clip):
    rng = np.random.default_rng(21 + clip)
    for H in (1024, 1030, 1056, 7168):
        xf = (rng.standard_normal(H) * rng.choice([1e-6, 1e-3, 1.0, 300.0], H)).astype(np.float32)
        xb = workloads.f32_to_bf16_bits(xf)
        xf = workloads.bf16_bits_to_f32(xb)
        codes, sc = oracle.quant_mx_row(xb, clip)
        nb = (H + 31) // 32
        assert len(sc) == nb + (nb & 1)
        assert (sc[nb:] == 0).all()
        for b in range(nb):
            blk = xf[b * 32:(b + 1) * 32]
            s = float(sc[b])
            m, e = math.frexp(s)
            assert m == 0.5                              # a power of two
            amax = float(np.abs(blk).max())
            se = e - 1
            if not clip:
                if amax > 0 and se > -127:
                    assert 256 <= amax / s < 512
            else:
                c = to_f32(Fraction(max(amax, float(np.float32(1e-4))))
                           / Fraction(448))
                assert 2.0 ** (se - 1) < c <= 2.0 ** se
            for v, code in zip(blk, codes[b * 32:(b + 1) * 32]):
                want = brute.e4m3_nearest(Fraction(float(v)) / Fraction(s))
                if want & 0x7F == 0 and v == 0:
                    want = 0x80 if math.copysign(1, float(v)) < 0 else 0
                assert code == want


def test_mx_matches_torch_float8_in_range():
    """Library special case: in-range values match torch's float8_e4m3fn cast."""
    import torch
    rng = np.random.default_rng(5)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal(4096).astype(np.float32))
    xf = workloads.bf16_bits_to_f32(xb)
    codes, sc = oracle.quant_mx_row(xb, clip=True)
    v = xf / np.repeat(sc[:128], 32)
    assert np.abs(v).max() <= 448
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (codes == want).all()


# ---------------------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------------------

def _single_rank_dispatch(W, E, BS, H, K, ids, mode=0):
    cfg = oracle.make_cfg(W, E, BS, H, K, quant_mode=mode)
    x = workloads.generate(workloads.C1_MODE0.replace(W=W, E=E, BS=BS, H=H, K=K), seed=4)["x"]
    d = oracle.dispatch(cfg, x, ids)
    return cfg, x, d


def test_combine_k1_unit_weight_is_the_row():
    W, E, BS, H, K = 2, 4, 3, 1024, 1
    ids = np.array([[[0], [3], [1]], [[2], [0], [0]]], np.int32)
    cfg, x, d = _single_rank_dispatch(W, E, BS, H, K, ids)
    w = np.ones((W, BS, K), np.float32)
    y = oracle.combine(cfg, d["expand_x"], ids, d["expand_idx"], w, d["ep_recv_count"],
                       d["recv_offsets"])
    assert (y == x).all()


def test_combine_exact_closed_form():
    """Power-of-two weights and small-integer rows: every fp32 step is exact, so
    y = sum_k w_k * row_k exactly."""
    W, E, BS, H, K = 2, 4, 2, 8, 3
    ids = np.array([[[0, 1, 2], [3, 0, 1]], [[1, 2, 3], [2, 0, 3]]], np.int32)
    cfg = oracle.make_cfg(W, E, BS, H, K)
    cnt, eidx = oracle.route(cfg, ids)
    erc, etn, off = oracle.recv_counts(cfg, cnt)
    P = int(off[-1])
    rows = np.arange(P * H, dtype=np.float32).reshape(P, H) % 17 - 8
    w = np.array([0.5, 0.25, 0.125], np.float32) * np.ones((W, BS, 1), np.float32)
    y = oracle.combine(cfg, bf16(rows), ids, eidx, w, erc, off)
    for s in range(W):
        for i in range(BS):
            want = np.zeros(H)
            for k in range(K):
                row = oracle.dest_row(cfg, erc, off, s, int(ids[s, i, k]), int(eidx[s, i, k]))
                want += float(w[s, i, k]) * rows[row]
            assert (workloads.bf16_bits_to_f32(y[s, i]) == want).all()


def test_combine_sums_in_k_order():
    """y = bf16 of the fp32 running sum over k = 0, 1, ..., K-1 of w_k * row_k ([DDD] §3.4.2):
    numpy float32 arithmetic in that order, rows located by the brute-force router.  Each
    token's first pick carries a large term that its last pick cancels exactly, with small
    terms between them, so the small terms are absorbed at the large term's spacing and the
    result depends on the order; the reverse order (a witness) gives a different y on the
    same draw.  Weights are powers of two, so every product is exact."""
    W, E, BS, H, K = 2, 8, 16, 1024, 6
    rng = np.random.default_rng(17)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(W * BS)]).astype(np.int32)
    ids = ids.reshape(W, BS, K)
    cfg = oracle.make_cfg(W, E, BS, H, K)
    cnt, eidx = oracle.route(cfg, ids)
    erc, etn, off = oracle.recv_counts(cfg, cnt)
    rows_of, *_ = brute.route(W, E, BS, K, ids)
    P = int(off[-1])
    w = rng.choice(np.float32([0.5, 1.0, 2.0]), (W, BS, K))
    v = rng.standard_normal((P, H)).astype(np.float32)
    big = np.float32(2.0 ** 16) * (1 + rng.random((W, BS, H))).astype(np.float32)
    big = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(big))
    for s in range(W):
        for i in range(BS):
            v[rows_of[(s, i, 0)]] = big[s, i]
            v[rows_of[(s, i, K - 1)]] = -big[s, i] * (w[s, i, 0] / w[s, i, K - 1])
    eo = workloads.f32_to_bf16_bits(v)
    rows = workloads.bf16_bits_to_f32(eo)
    assert (rows[[rows_of[(s, i, K - 1)] for s in range(W) for i in range(BS)]]
            == -(big * (w[..., :1] / w[..., K - 1:])).reshape(W * BS, H)).all()
    y = oracle.combine(cfg, eo, ids, eidx, w, erc, off)
    differs = 0
    for s in range(W):
        for i in range(BS):
            terms = [w[s, i, k] * rows[rows_of[(s, i, k)]] for k in range(K)]
            fwd = np.zeros(H, np.float32)
            for t in terms:
                fwd = fwd + t
            rev = np.zeros(H, np.float32)
            for t in reversed(terms):
                rev = rev + t
            want = workloads.f32_to_bf16_bits(fwd)
            assert (y[s, i] == want).all(), (s, i)
            differs += int((workloads.f32_to_bf16_bits(rev) != want).sum())
    assert differs > 1000, f"the draw should make the summation order visible ({differs})"


def test_combine_special_experts_and_masks():
    W, E, BS, H, K = 2, 4, 3, 1024, 2
    Z, C = 1, 1
    ids = np.array([[[0, 4], [5, 1], [4, 5]], [[2, 3], [5, 5], [0, 1]]], np.int32)
    mask = np.array([[[1, 1], [1, 1], [1, 1]], [[1, 1], [1, 0], [0, 0]]], np.uint8)
    cfg = oracle.make_cfg(W, E, BS, H, K, zero_expert_num=Z, copy_expert_num=C, mask_kind=2)
    x = workloads.generate(workloads.C1_MODE0.replace(W=W, E=E, BS=BS, H=H, K=K), seed=2)["x"]
    d = oracle.dispatch(cfg, x, ids, mask=mask)
    # routed picks: (0,0,0) (0,1,1) (1,0,0) (1,0,1); the rest are special or masked
    assert d["recv_offsets"][-1] == 4
    w = np.array([[[0.5, 0.25], [1.0, 2.0], [0.5, 0.5]], [[1, 1], [0.5, 3.0], [1, 1]]],
                 np.float32)
    y = oracle.combine(cfg, d["expand_x"], ids, d["expand_idx"], w, d["ep_recv_count"],
                       d["recv_offsets"], mask=mask, ori_x=x)
    xf = workloads.bf16_bits_to_f32(x)
    yf = workloads.bf16_bits_to_f32(y)
    # token (0,0): expert 0 (routed, identity) * 0.5 + zero expert -> 0.5 x
    assert (yf[0, 0] == 0.5 * xf[0, 0]).all()
    # token (0,1): copy expert * 1.0 + expert 1 * 2.0 -> 3 x (bf16-rounded)
    assert (y[0, 1] == workloads.f32_to_bf16_bits(xf[0, 1] + 2.0 * xf[0, 1])).all()
    # token (0,2): zero + copy*0.5 -> 0.5 x
    assert (yf[0, 2] == 0.5 * xf[0, 2]).all()
    # token (1,1): second pick masked off -> copy * 0.5
    assert (yf[1, 1] == 0.5 * xf[1, 1]).all()
    # token (1,2): fully inactive -> +0
    assert (y[1, 2] == 0).all()


def test_combine_roundtrip_identity_ffn():
    """Mode 0 with an identity expert and softmax weights: y ~ x within bf16 rounding and
    the fp32 error of the weights' sum (the weights sum to 1 up to a few ulps)."""
    wl = workloads.C1_MODE0
    inp = workloads.generate(wl, seed=0)
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K)
    d = oracle.dispatch(cfg, inp["x"], inp["expert_ids"])
    y = oracle.combine(cfg, d["expand_x"], inp["expert_ids"], d["expand_idx"],
                       inp["expert_scales"], d["ep_recv_count"], d["recv_offsets"])
    xf = workloads.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    yf = workloads.bf16_bits_to_f32(y).astype(np.float64)
    assert (np.abs(yf - xf) <= np.abs(xf) * (2.0 ** -8 + 2.0 ** -20)).all()


def test_combine_roundtrip_int8():
    """Mode 2 then an identity-dequant expert (bf16(q * scale)): the error per element is
    at most half an int8 step plus bf16 rounding, weighted by the picks' weights."""
    wl = workloads.C1_MODE2
    inp = workloads.generate(wl, seed=1)
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, quant_mode=2)
    d = oracle.dispatch(cfg, inp["x"], inp["expert_ids"])
    P = int(d["recv_offsets"][-1])
    deq = d["expand_x"][:P].astype(np.float32) * d["dynamic_scales"][:P, None]
    eo = workloads.f32_to_bf16_bits(deq)
    y = oracle.combine(cfg, eo, inp["expert_ids"], d["expand_idx"], inp["expert_scales"],
                       d["ep_recv_count"], d["recv_offsets"])
    xf = workloads.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    yf = workloads.bf16_bits_to_f32(y).astype(np.float64)
    amax = np.abs(xf).max(axis=2, keepdims=True)
    bound = 0.5 * amax / 127 + np.abs(xf) * 2.0 ** -7 + amax * 2.0 ** -8
    assert (np.abs(yf - xf) <= bound).all()


# ---------------------------------------------------------------------------------------
# whole dispatch: payload placement against brute-force rows
# ---------------------------------------------------------------------------------------

VARIANTS = [  # (quant_mode, out_dtype, scales_kind, scale_format)
    (0, 0, 0, 0), (1, 0, 1, 0), (1, 1, 2, 0), (1, 0, 3, 0), (2, 0, 0, 0), (2, 0, 3, 0),
    (2, 2, 2, 0), (2, 3, 1, 0), (3, 0, 0, 0), (3, 3, 3, 0), (4, 0, 0, 0), (4, 3, 0, 1),
    (5, 0, 0, 0), (5, 2, 0, 1), (5, 3, 0, 0), (4, 4, 0, 0), (5, 4, 0, 1), (4, 0, 0, 2),
    (5, 4, 0, 2)]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: "m%d_t%d_s%d_f%d" % v)
def test_dispatch_payload_placement(variant):
    mode, odt, kind, fmt = variant
    wl = workloads.C1_MODE0.replace(quant_mode=mode, zero_expert_num=1, copy_expert_num=1,
                                    mask_kind=2, inactive_tokens_per_rank=3, routing="randint",
                                    out_dtype=odt, scales_kind=kind, scale_format=fmt)
    inp = workloads.generate(wl, seed=9)
    sm = inp["scales"]
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, quant_mode=mode,
                          zero_expert_num=1, copy_expert_num=1, mask_kind=2, out_dtype=odt,
                          scales_kind=kind, scale_format=fmt)
    d = oracle.dispatch(cfg, inp["x"], inp["expert_ids"], scales=sm, mask=inp["mask"])
    rows, beidx, *_ = brute.route(wl.W, wl.E, wl.BS, wl.K, inp["expert_ids"].tolist(),
                                  inp["mask"].tolist(), 2)
    assert d["expand_idx"].tolist() == beidx
    assert int(d["recv_offsets"][-1]) == len(rows)
    for (s, i, k), row in rows.items():
        assert d["assist_info"][row].tolist() == [s, i, k]
        xr = inp["x"][s, i]
        if mode == 0:
            assert (d["expand_x"][row] == xr).all()
            continue
        pre = None if kind == 0 else sm[inp["expert_ids"][s, i, k]] if kind == 3 else sm
        q, sc = oracle.quant_row(mode, xr, pre, odt)
        assert (d["expand_x"][row] == q).all()
        if mode == 1:
            assert "dynamic_scales" not in d
        elif fmt == 1:
            nb = (wl.H + 31) // 32
            want = [oracle.e8m0_from_scale(v) for v in sc[:nb]] + [0] * (len(sc) - nb)
            assert d["dynamic_scales"][row].tolist() == want
        elif fmt == 2:
            # the formula's literal transmitted value, 1.0 / dynamic_scales_value ([LLD]
            # 计算公式, modes 4/5), of a power of two: exact in binary64 and in binary32
            nb = (wl.H + 31) // 32
            want = np.array([1.0 / float(v) for v in sc[:nb]] + [0.0] * (len(sc) - nb),
                            np.float32)
            assert (d["dynamic_scales"][row].view(np.uint32) == want.view(np.uint32)).all()
        else:
            assert (d["dynamic_scales"][row] == sc).all()


@pytest.mark.parametrize("variant", [(0, 2, 0, 0), (1, 0, 0, 0), (1, 2, 1, 0), (2, 0, 0, 1),
                                     (3, 1, 0, 0), (4, 0, 1, 0), (5, 1, 0, 0), (3, 0, 4, 0),
                                     (2, 0, 0, 2), (3, 0, 0, 2), (4, 0, 0, 3)])
def test_dispatch_rejects_invalid_variants(variant):
    mode, odt, kind, fmt = variant
    cfg = oracle.make_cfg(2, 8, 4, 1024, 2, quant_mode=mode, out_dtype=odt, scales_kind=kind,
                          scale_format=fmt)
    x = np.zeros((2, 4, 1024), np.uint16)
    ids = np.zeros((2, 4, 2), np.int32)
    sc = None if kind == 0 else np.ones(1024, np.float32)
    with pytest.raises(ValueError):
        oracle.dispatch(cfg, x, ids, scales=sc)


@pytest.mark.parametrize("mode", [4, 5])
def test_mx_reciprocal_scales_with_pad(mode):
    """scale_format 2 on a row with an odd block count (H = 1056: 33 blocks, Align2 -> 34): each
    block's entry is 1 / 2^shared_exp, i.e. the entry of scale_format 0 inverted (exact for a
    power of two), codes unchanged, the pad entry 0; and x is the codes divided by the
    transmitted value, within half an E4M3 step."""
    wl = workloads.Workload("mx_recip", W=2, E=4, BS=5, H=1056, K=2, quant_mode=mode)
    inp = workloads.generate(wl, seed=4)
    out = {}
    for fmt in (0, 2):
        cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, quant_mode=mode, scale_format=fmt)
        out[fmt] = oracle.dispatch(cfg, inp["x"], inp["expert_ids"])
    P = int(out[0]["recv_offsets"][-1])
    a, b = out[0]["dynamic_scales"][:P], out[2]["dynamic_scales"][:P]
    assert (out[0]["expand_x"][:P] == out[2]["expand_x"][:P]).all()
    assert (b[:, 33] == 0).all() and (a[:, 33] == 0).all()
    assert (a[:, :33].astype(np.float64) * b[:, :33].astype(np.float64) == 1.0).all()
    for row in range(P):
        s, i, _ = out[2]["assist_info"][row]
        xf = workloads.bf16_bits_to_f32(inp["x"][s, i]).astype(np.float64)
        codes = np.array([oracle.e4m3_to_f32(c) for c in out[2]["expand_x"][row]], np.float64)
        recon = codes / np.repeat(b[row, :33].astype(np.float64), 32)[:wl.H]
        step = np.repeat(1.0 / b[row, :33].astype(np.float64), 32)[:wl.H]
        # E4M3 spacing relative to the element: at most 2^-3 of the value, or the subnormal step
        tol = np.maximum(np.abs(xf) * 2.0 ** -4, step * 2.0 ** -10)
        clip = np.abs(xf) >= 448 * step              # saturated elements (mode 4 overflow)
        assert (np.abs(recon - xf)[~clip] <= tol[~clip]).all()
