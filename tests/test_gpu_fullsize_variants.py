"""GPU parity of the quantization and combine variants at full workload sizes, in the
library's normal launch configuration.  Every output is compared in full against the oracle
run over the whole workload: routing outputs and every routed row of expand_x,
dynamic_scales and assist_info bit for bit; combine-side int8 codes and block scales of every
routed row bit for bit; every element of y within 1e-2 relative / 1e-3 absolute (and
asserted bit-identical)."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

DISPATCH_CASES = {
    # the W=32, H=8192, K=16 shape with MXFP4 clip codes and E8M0 scales
    "c5_mxfp4_e8m0": workloads.C5.replace(name="c5v_mxfp4_e8m0", out_dtype=4, scale_format=1),
    # per-128-group E4M3 with per-expert smooth scales at the W=16, H=7168 shape
    "c4_group_smooth": workloads.C4.replace(name="c4v_group_smooth", quant_mode=3,
                                            scales_kind=3),
    # per-token int8 with per-expert smooth scales at the W=16, H=7168 shape
    "c4_smooth": workloads.C4_SMOOTH,
    # MX E5M2 + E8M0 at the Zipf-routed W=16 shape
    "c3_e5m2_e8m0": workloads.C3_E5M2_E8M0,
    # int8 per token at the W=16, H=7168 shape with binary16 tokens
    "c4_f16_tokens": workloads.C4_F16,
}


def _check_y(tag, y_dev, y_ref, token_dtype=0):
    y = harness.host(y_dev)
    ndiff = harness.check_combine_tolerance(y.reshape(y_ref.shape), y_ref,
                                            token_dtype=token_dtype)
    print(f"[{tag}] y: {y_ref.size - ndiff} of {y_ref.size} elements bit-identical",
          flush=True)
    assert ndiff == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(DISPATCH_CASES))
def test_fullsize_variant_dispatch(name):
    import torch
    wl = DISPATCH_CASES[name]
    inp = workloads.generate(wl, seed=0)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)        # every routed row, bit for bit
    print(f"[{name}] dispatch: {int(ref['recv_offsets'][-1])} routed rows identical",
          flush=True)


@pytest.mark.timeout(900)
def test_c5_int8_combine_fullsize():
    """W=32, H=8192, K=16 (8-element lanes: K > 8) with special experts and masks: the
    expert-side codes and block scales of every routed row, and every element of y, against
    the oracle."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C5
    inp = workloads.generate(wl, seed=0)
    ocfg = harness.oracle_cfg(wl)
    cnt, eidx = oracle.route(ocfg, inp["expert_ids"], inp.get("mask"))
    erc, etn, off = oracle.recv_counts(ocfg, cnt)
    P = int(off[-1])
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo_dev = workloads.expert_out_torch(wl, wl.cap, seed=0)
    codes, scales = cq.combine_quantize(cfg, eo_dev, out["recv_offsets"])
    y = cq.combine_int8(cfg, codes, scales, dev_in["ids"], out["expand_idx"],
                        harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                        out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(harness.host(out["expand_idx"]), eidx)
    np.testing.assert_array_equal(harness.host(out["ep_recv_count"]), erc)
    np.testing.assert_array_equal(harness.host(out["recv_offsets"]), off)
    eo_h = harness.host(eo_dev)
    del eo_dev
    codes_ref, scales_ref = oracle.combine_quantize(ocfg, eo_h, off)
    del eo_h
    np.testing.assert_array_equal(harness.host(codes[:P]), codes_ref[:P], err_msg="codes")
    np.testing.assert_array_equal(harness.host(scales[:P]).view(np.uint32),
                                  scales_ref[:P].view(np.uint32), err_msg="block scales")
    print(f"[c5 int8 combine] codes and scales of {P} routed rows identical", flush=True)
    y_ref = oracle.combine_int8(ocfg, codes_ref, scales_ref, inp["expert_ids"], eidx,
                                inp["expert_scales"], erc, off, mask=inp["mask"],
                                ori_x=inp["x"])
    _check_y("c5 int8 combine", y, y_ref)


@pytest.mark.timeout(900)
def test_c4_f16_combine_fullsize():
    """The W=16, H=7168, K=8 round trip with binary16 tokens at full size: every element of
    the gather combine's output against the oracle, from the rows it reads."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C4_F16
    inp = workloads.generate(wl, seed=0)
    ocfg = harness.oracle_cfg(wl)
    cnt, eidx = oracle.route(ocfg, inp["expert_ids"], inp.get("mask"))
    erc, etn, off = oracle.recv_counts(ocfg, cnt)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo_dev = workloads.expert_out_torch(wl, wl.cap, seed=0)
    assert eo_dev.dtype == torch.float16
    y = cq.combine(cfg, eo_dev, dev_in["ids"], out["expand_idx"],
                   harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                   out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    np.testing.assert_array_equal(harness.host(out["expand_idx"]), eidx)
    eo_h = harness.host(eo_dev)
    del eo_dev
    y_ref = oracle.combine(ocfg, eo_h, inp["expert_ids"], eidx, inp["expert_scales"], erc,
                           off, mask=inp.get("mask"), ori_x=inp["x"])
    _check_y("c4 f16 combine", y, y_ref, token_dtype=1)
