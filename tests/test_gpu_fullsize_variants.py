"""GPU parity of the quantization and combine variants at full workload sizes, in the
library's normal launch configuration: routing outputs and the packed layout in full,
payload rows and combine outputs of seeded sample tokens recomputed one by one by the
oracle."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

N_SAMPLE = 96

DISPATCH_CASES = {
    # the W=32, H=8192, K=16 shape with MXFP4 clip codes and E8M0 scales
    "c5_mxfp4_e8m0": workloads.C5.replace(name="c5v_mxfp4_e8m0", out_dtype=4, scale_format=1),
    # per-128-group E4M3 with per-expert smooth scales at the W=16, H=7168 shape
    "c4_group_smooth": workloads.C4.replace(name="c4v_group_smooth", quant_mode=3,
                                            scales_kind=3),
    # MX E5M2 + E8M0 at the Zipf-routed W=16 shape
    "c3_e5m2_e8m0": workloads.C3_E5M2_E8M0,
    # int8 per token at the W=16, H=7168 shape with binary16 tokens
    "c4_f16_tokens": workloads.C4_F16,
}


def _sample(wl, seed):
    rng = np.random.default_rng(seed)
    flat = np.sort(rng.choice(wl.T, size=min(N_SAMPLE, wl.T), replace=False))
    return [(int(f) // wl.BS, int(f) % wl.BS) for f in flat]


@pytest.mark.parametrize("name", list(DISPATCH_CASES))
def test_fullsize_variant_dispatch(name):
    import torch
    wl = DISPATCH_CASES[name]
    inp = workloads.generate(wl, seed=0)
    ocfg = harness.oracle_cfg(wl)
    cnt, eidx = oracle.route(ocfg, inp["expert_ids"], inp.get("mask"))
    erc, etn, off = oracle.recv_counts(ocfg, cnt)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(harness.host(out["expand_idx"]), eidx)
    np.testing.assert_array_equal(harness.host(out["ep_recv_count"]), erc)
    np.testing.assert_array_equal(harness.host(out["expert_token_nums"]), etn)
    np.testing.assert_array_equal(harness.host(out["recv_offsets"]), off)
    ct = oracle.code_type(wl.quant_mode, wl.out_dtype)
    nb = (wl.H + 31) // 32
    ai = harness.host(out["assist_info"])
    for s, i in _sample(wl, 11):
        for k in range(wl.K):
            o = int(eidx[s, i, k])
            if o < 0:
                continue
            e = int(inp["expert_ids"][s, i, k])
            row = int(oracle.dest_row(ocfg, erc, off, s, e, o))
            assert tuple(ai[row]) == (s, i, k)
            pre = None if wl.scales_kind == 0 else inp["scales"][e]
            q, sc = oracle.quant_row(wl.quant_mode, inp["x"][s, i], pre, wl.out_dtype,
                                     token_dtype=wl.token_dtype)
            got = harness.host(out["expand_x"][row])
            assert (got.view(np.uint8) == q.view(np.uint8)).all(), (s, i, k)
            ds = harness.host(out["dynamic_scales"][row])
            if wl.scale_format == 1:
                want = [oracle.e8m0_from_scale(v) for v in sc[:nb]] + [0] * (len(sc) - nb)
                assert ds.tolist() == want, (s, i, k)
            else:
                assert (ds.view(np.uint32) == sc.view(np.uint32)).all(), (s, i, k)
    assert ct >= 0


def test_c5_int8_combine_sampled():
    """W=32, H=8192, K=16 (8-element lanes: K > 8) with special experts and masks: sampled
    rows' codes and scales, and sampled tokens' outputs, against the oracle."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C5
    inp = workloads.generate(wl, seed=0)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo_dev = workloads.expert_out_torch(wl, wl.cap, seed=0)
    codes, scales = cq.combine_quantize(cfg, eo_dev, out["recv_offsets"])
    y = cq.combine_int8(cfg, codes, scales, dev_in["ids"], out["expand_idx"],
                        harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                        out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    eidx = harness.host(out["expand_idx"])
    erc = harness.host(out["ep_recv_count"])
    roff = harness.host(out["recv_offsets"])
    ocfg = harness.oracle_cfg(wl)
    tokens = _sample(wl, 5)
    rows = sorted({int(oracle.dest_row(ocfg, erc, roff, s, int(inp["expert_ids"][s, i, k]),
                                       int(eidx[s, i, k])))
                   for s, i in tokens for k in range(wl.K) if eidx[s, i, k] >= 0})
    rows_t = torch.tensor(rows, dtype=torch.long, device="cuda")
    eo_rows = harness.host(eo_dev.index_select(0, rows_t))
    c_rows = harness.host(codes.index_select(0, rows_t))
    s_rows = harness.host(scales.index_select(0, rows_t))
    codes_h = np.zeros((wl.cap, wl.H), np.int8)
    scales_h = np.zeros((wl.cap, (wl.H + 7) // 8), np.float32)
    for n, r in enumerate(rows):
        q, sc = oracle.combine_quant_row(eo_rows[n])
        assert (c_rows[n] == q).all() and (s_rows[n].view(np.uint32) == sc.view(np.uint32)).all()
        codes_h[r], scales_h[r] = q, sc
    y_h = harness.host(y)
    for s, i in tokens:
        want = oracle.combine_int8_token(ocfg, codes_h, scales_h, inp["expert_ids"], eidx,
                                         inp["expert_scales"], erc, roff, s, i,
                                         mask=inp["mask"], ori_x=inp["x"])
        assert harness.check_combine_tolerance(y_h[s, i], want) == 0


def test_c4_f16_combine_sampled():
    """The W=16, H=7168, K=8 round trip with binary16 tokens at full size: the gather
    combine's outputs for sampled tokens against the oracle, from the rows they read."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C4_F16
    inp = workloads.generate(wl, seed=0)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo_dev = workloads.expert_out_torch(wl, wl.cap, seed=0)
    assert eo_dev.dtype == torch.float16
    y = cq.combine(cfg, eo_dev, dev_in["ids"], out["expand_idx"],
                   harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                   out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    eidx = harness.host(out["expand_idx"])
    erc = harness.host(out["ep_recv_count"])
    roff = harness.host(out["recv_offsets"])
    ocfg = harness.oracle_cfg(wl)
    tokens = _sample(wl, 7)
    rows = sorted({int(oracle.dest_row(ocfg, erc, roff, s, int(inp["expert_ids"][s, i, k]),
                                       int(eidx[s, i, k])))
                   for s, i in tokens for k in range(wl.K) if eidx[s, i, k] >= 0})
    rows_t = torch.tensor(rows, dtype=torch.long, device="cuda")
    eo_rows = harness.host(eo_dev.index_select(0, rows_t))
    eo_h = np.zeros((wl.cap, wl.H), np.uint16)
    eo_h[rows] = eo_rows
    y_h = harness.host(y)
    for s, i in tokens:
        want = oracle.combine_token(ocfg, eo_h, inp["expert_ids"], eidx, inp["expert_scales"],
                                    erc, roff, s, i, mask=inp.get("mask"), ori_x=inp["x"])
        assert harness.check_combine_tolerance(y_h[s, i], want, token_dtype=1) == 0, (s, i)
