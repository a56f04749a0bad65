"""Pins of the CPU oracle with IEEE binary16 tokens (the pages allow float16 as well as
bfloat16 for x, the expert outputs and y; CPU only).

The quantization and the combine sum work on the fp32 value of each element, so binary16
tokens are pinned through numpy's own float16 conversions (widening exact, narrowing to
nearest even) and through rows whose values both formats hold exactly, which must give the
same codes, scales and sums whichever type carries them.
"""
import numpy as np
import pytest

import oracle
import workloads

F16 = oracle.TOKEN_F16


def f16(vals):
    return np.asarray(vals, np.float32).astype(np.float16).view(np.uint16)


def _shared_values(rng, H):
    """Values exact in both bf16 and binary16: integers of magnitude < 256 times 2^e,
    e in [-6, 4] (at most 8 significant bits, inside binary16's normal range)."""
    m = rng.integers(-255, 256, H).astype(np.float32)
    e = rng.integers(-6, 5, H).astype(np.float32)
    return m * np.exp2(e).astype(np.float32)


def test_f16_int8_row_is_numpy_float32():
    """Mode 2 without smooth scales on binary16 rows: numpy float32 division, multiply,
    rint on the exactly widened values."""
    rng = np.random.default_rng(11)
    for scale in (1.0, 1e-3, 300.0):
        xh = f16(rng.standard_normal(4096) * scale)
        xf = xh.view(np.float16).astype(np.float32)
        q, sc = oracle.quant_row(2, xh, token_dtype=F16)
        dyn = np.float32(127) / np.max(np.abs(xf))
        assert (q == np.rint(xf * dyn).astype(np.int8)).all()
        assert sc[0] == np.float32(1) / dyn


@pytest.mark.parametrize("mode,out_dtype", [(1, 0), (2, 0), (2, 2), (3, 2), (3, 3), (4, 0),
                                            (4, 3), (4, 4), (5, 0), (5, 4)])
def test_same_values_quantize_alike_in_both_token_types(mode, out_dtype):
    rng = np.random.default_rng(mode * 10 + out_dtype)
    H = 1056
    v = _shared_values(rng, H)
    xb, xh = workloads.f32_to_bf16_bits(v), f16(v)
    assert (workloads.bf16_bits_to_f32(xb) == v).all() and (xh.view(np.float16) == v).all()
    pre = np.full(1, 0.25, np.float32) if mode == 1 else None
    qb, sb = oracle.quant_row(mode, xb, pre, out_dtype=out_dtype)
    qh, sh = oracle.quant_row(mode, xh, pre, out_dtype=out_dtype, token_dtype=F16)
    assert (qb == qh).all()
    assert (sb.view(np.uint32) == sh.view(np.uint32)).all()


def test_combine_quant_row_same_values_alike():
    rng = np.random.default_rng(5)
    v = _shared_values(rng, 1032)
    qb, sb = oracle.combine_quant_row(workloads.f32_to_bf16_bits(v))
    qh, sh = oracle.combine_quant_row(f16(v), token_dtype=F16)
    assert (qb == qh).all() and (sb.view(np.uint32) == sh.view(np.uint32)).all()


def _f16_dispatch(ids, W, E, BS, H, K, mode=0, seed=4):
    cfg = oracle.make_cfg(W, E, BS, H, K, quant_mode=mode, token_dtype=F16)
    wl = workloads.C1_MODE0.replace(W=W, E=E, BS=BS, H=H, K=K, token_dtype=1)
    x = workloads.generate(wl, seed=seed)["x"]
    return cfg, x, oracle.dispatch(cfg, x, ids)


def test_mode0_moves_binary16_rows_unchanged():
    W, E, BS, H, K = 2, 4, 3, 1024, 2
    ids = np.array([[[0, 3], [1, 2], [3, 0]], [[2, 1], [0, 3], [1, 0]]], np.int32)
    cfg, x, d = _f16_dispatch(ids, W, E, BS, H, K)
    P = int(d["recv_offsets"][-1])
    for r in range(P):
        s, i, _ = d["assist_info"][r]
        assert (d["expand_x"][r].view(np.uint16) == x[s, i]).all()


def test_combine_k1_unit_weight_is_the_binary16_row():
    W, E, BS, H, K = 2, 4, 3, 1024, 1
    ids = np.array([[[0], [3], [1]], [[2], [0], [0]]], np.int32)
    cfg, x, d = _f16_dispatch(ids, W, E, BS, H, K)
    w = np.ones((W, BS, K), np.float32)
    y = oracle.combine(cfg, d["expand_x"], ids, d["expand_idx"], w, d["ep_recv_count"],
                       d["recv_offsets"])
    assert (y == x).all()


def test_combine_sum_rounds_to_binary16_like_numpy():
    """y = binary16(fp32 sum over picks in k order of w * row): numpy float32 arithmetic in
    the same order, then numpy's float16 cast (nearest even, overflow to inf)."""
    W, E, BS, H, K = 2, 4, 3, 1024, 2
    ids = np.array([[[0, 3], [1, 2], [3, 0]], [[2, 1], [0, 3], [1, 0]]], np.int32)
    cfg, x, d = _f16_dispatch(ids, W, E, BS, H, K)
    rng = np.random.default_rng(9)
    cap = W * BS * K
    eo_f = (rng.standard_normal((cap, H)) * 3000).astype(np.float32)
    eo = f16(eo_f)
    w = rng.random((W, BS, K)).astype(np.float32) * 20
    y = oracle.combine(cfg, eo, ids, d["expand_idx"], w, d["ep_recv_count"], d["recv_offsets"])
    rows = {}
    for r in range(int(d["recv_offsets"][-1])):
        s, i, k = d["assist_info"][r]
        rows[(s, i, k)] = r
    eo_w = eo.view(np.float16).astype(np.float32)
    for s in range(W):
        for i in range(BS):
            acc = np.zeros(H, np.float32)
            for k in range(K):
                acc = acc + w[s, i, k] * eo_w[rows[(s, i, k)]]
            with np.errstate(over="ignore"):
                ref = acc.astype(np.float16).view(np.uint16)
            assert (y[s, i] == ref).all(), (s, i)
    assert np.isinf(y.view(np.float16)).any(), "the draw should reach binary16 overflow"
