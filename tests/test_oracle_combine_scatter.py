"""Pins of the oracle's row weights (expand_scales) and scatter-back combine against what
the pages fix, independently of the functions under test:

  * expand_scales: each dispatched row carries the weight of the pick brute force places in
    that row;
  * the scatter-back combine (rows sent back by their assist_info triples to slot
    i*K + k, then a per-token K-sum) equals the separately pinned gather combine, whose
    addresses come from expand_idx and ep_recv_count instead, on random tiny configurations
    with masks, special experts and duplicate picks;
  * the shared expert's output: alone when every pick is inactive, and added after the K
    picks (a closed-form case where the other order gives a different bf16).
"""
import numpy as np
import pytest

import brute
import oracle
import workloads


def _case(seed, **kw):
    wl = workloads.C1_MODE0.replace(**kw)
    inp = workloads.generate(wl, seed=seed)
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, zero_expert_num=wl.zero_expert_num,
                          copy_expert_num=wl.copy_expert_num, mask_kind=wl.mask_kind)
    d = oracle.dispatch(cfg, inp["x"], inp["expert_ids"], mask=inp.get("mask"))
    return wl, cfg, inp, d


CONFIGS = [
    dict(),
    dict(W=4, E=16, BS=9, K=4, routing="randint"),
    dict(W=3, E=12, BS=7, K=5, zero_expert_num=1, copy_expert_num=2, mask_kind=2,
         inactive_tokens_per_rank=2, routing="randint"),
    dict(W=2, E=4, BS=11, K=6, zero_expert_num=1, copy_expert_num=1, mask_kind=1,
         inactive_tokens_per_rank=3, routing="randint"),
    dict(W=4, E=32, BS=5, K=16, routing="uniform"),
]


@pytest.mark.parametrize("idx", range(len(CONFIGS)))
def test_expand_scales_follow_the_brute_force_rows(idx):
    wl, cfg, inp, d = _case(idx, **CONFIGS[idx])
    es = oracle.expand_scales(cfg, d["assist_info"], d["recv_offsets"], inp["expert_scales"],
                              wl.cap)
    mask = None if inp.get("mask") is None else inp["mask"].tolist()
    rows, *_ = brute.route(wl.W, wl.E, wl.BS, wl.K, inp["expert_ids"].tolist(), mask,
                           wl.mask_kind)
    assert len(rows) == int(d["recv_offsets"][-1])
    for (s, i, k), r in rows.items():
        assert es[r] == inp["expert_scales"][s, i, k]
    assert (es[len(rows):] == 0).all()


@pytest.mark.parametrize("idx", range(len(CONFIGS)))
@pytest.mark.parametrize("seed", [0, 1])
def test_scatter_back_equals_the_gather_combine(idx, seed):
    wl, cfg, inp, d = _case(10 * idx + seed, **CONFIGS[idx])
    eo = workloads.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(
        (wl.cap, wl.H)).astype(np.float32))
    y_g = oracle.combine(cfg, eo, inp["expert_ids"], d["expand_idx"], inp["expert_scales"],
                         d["ep_recv_count"], d["recv_offsets"], mask=inp.get("mask"),
                         ori_x=inp["x"])
    y_s = oracle.combine_scatter(cfg, eo, d["assist_info"], d["recv_offsets"],
                                 inp["expert_ids"], inp["expert_scales"],
                                 mask=inp.get("mask"), ori_x=inp["x"])
    assert (y_g == y_s).all()


def test_shared_term_alone_when_every_pick_is_inactive():
    wl, cfg, inp, d = _case(3, mask_kind=1, inactive_tokens_per_rank=16)
    assert int(d["recv_offsets"][-1]) == 0
    shared = workloads.f32_to_bf16_bits(np.random.default_rng(2).standard_normal(
        (wl.W, wl.BS, wl.H)).astype(np.float32))
    y = oracle.combine_scatter(cfg, np.zeros((wl.cap, wl.H), np.uint16), d["assist_info"],
                               d["recv_offsets"], inp["expert_ids"], inp["expert_scales"],
                               mask=inp["mask"], shared_x=shared)
    assert (y == shared).all()


def test_shared_term_is_added_after_the_picks():
    """K=3 picks with weight 1 and values 2^-24, 1, 2^-8 (in k order), shared 2^-24.
    Picks first: 2^-24 + 1 rounds to 1 (tie to even), + 2^-8 = 1 + 2^-8, + 2^-24 rounds back
    (tie to even): exactly the bf16 midpoint 1 + 2^-8, which rounds to 1.0.  With the shared
    value first, 2^-24 + 2^-24 + 1 + 2^-8 = 1 + 2^-8 + 2^-23 exactly, which rounds to
    1 + 2^-7: the test tells the two orders apart."""
    W, E, BS, H, K = 2, 6, 1, 1024, 3
    cfg = oracle.make_cfg(W, E, BS, H, K)
    ids = np.array([[[0, 1, 2]], [[3, 4, 5]]], np.int32)
    x = np.zeros((W, BS, H), np.uint16)
    d = oracle.dispatch(cfg, x, ids)
    eo = np.zeros((W * BS * K, H), np.uint16)
    vals = [2.0 ** -24, 1.0, 2.0 ** -8]
    for s in range(W):
        for k in range(K):
            row = oracle.dest_row(cfg, d["ep_recv_count"], d["recv_offsets"], s, ids[s, 0, k],
                                  d["expand_idx"][s, 0, k])
            eo[row] = workloads.f32_to_bf16_bits(np.full(H, vals[k], np.float32))
    w = np.ones((W, BS, K), np.float32)
    shared = workloads.f32_to_bf16_bits(np.full((W, BS, H), 2.0 ** -24, np.float32))
    y = oracle.combine_scatter(cfg, eo, d["assist_info"], d["recv_offsets"], ids, w,
                               shared_x=shared)
    assert (workloads.bf16_bits_to_f32(y) == 1.0).all()
    y0 = oracle.combine_scatter(cfg, eo, d["assist_info"], d["recv_offsets"], ids, w)
    assert (workloads.bf16_bits_to_f32(y0) == 1.0).all()


def test_rejects_a_triple_out_of_range():
    wl, cfg, inp, d = _case(4)
    bad = d["assist_info"].copy()
    bad[0, 1] = wl.BS
    with pytest.raises(ValueError):
        oracle.combine_scatter(cfg, np.zeros((wl.cap, wl.H), np.uint16), bad,
                               d["recv_offsets"], inp["expert_ids"], inp["expert_scales"])
