"""GPU parity with IEEE binary16 tokens (cfg token_dtype = MOE_TOKEN_F16): x, the expert
outputs, ori_x, the shared expert's output and y in binary16.  Dispatch against the oracle
bit for bit, every combine within 1e-2 relative / 1e-3 absolute per binary16 element of the
oracle (expected bit-identical), through the C ABI, on the vectorized and element-wise
kernels and on both routing paths."""
import numpy as np
import pytest

import combine_quant_amd as cq
import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload

CASES = {
    "c1_mode0": workloads.C1_MODE0.replace(name="f16_c1_mode0", token_dtype=1),
    "c1_mode2": workloads.C1_MODE2.replace(name="f16_c1_mode2", token_dtype=1),
    "static_shared": WL("f16_static", W=4, E=16, BS=40, H=1024, K=4, quant_mode=1,
                        scales_kind=2, token_dtype=1),
    "smooth_per_expert": WL("f16_smooth", W=4, E=32, BS=70, H=2048, K=8, quant_mode=2,
                            scales_kind=3, outlier_prob=0.02, token_dtype=1),
    # past the pick kernel's limit: one workgroup per (window of tokens, expert)
    "smooth_windows": WL("f16_smooth_windows", W=8, E=64, BS=272, H=1032, K=8, quant_mode=2,
                         scales_kind=3, outlier_prob=0.02, token_dtype=1),
    "group_smooth_windows": WL("f16_group_windows", W=8, E=32, BS=352, H=1160, K=6,
                               quant_mode=3, out_dtype=2, scales_kind=3, mask_kind=2,
                               inactive_tokens_per_rank=20, token_dtype=1),
    "group_e5m2_ragged": WL("f16_group", W=4, E=32, BS=50, H=1056, K=6, quant_mode=3,
                            out_dtype=3, token_dtype=1),
    "mx_e4m3_zipf": WL("f16_mx", W=8, E=64, BS=64, H=7168, K=8, quant_mode=4,
                       routing="zipf", token_dtype=1),
    "mx_clip_fp4_special": WL("f16_mxclip", W=4, E=32, BS=60, H=2048, K=16, quant_mode=5,
                              out_dtype=4, scale_format=1, zero_expert_num=2,
                              copy_expert_num=2, mask_kind=2, inactive_tokens_per_rank=6,
                              token_dtype=1),
    "int8_h7168": WL("f16_int8", W=8, E=64, BS=128, H=7168, K=8, quant_mode=2,
                     copy_expert_num=1, routing="randint", token_dtype=1),
    "elementwise_h1030": WL("f16_h1030", W=2, E=8, BS=33, H=1030, K=3, quant_mode=2,
                            copy_expert_num=1, mask_kind=1, inactive_tokens_per_rank=4,
                            token_dtype=1),
}


@pytest.mark.parametrize("flags", [0, cq.MOE_DC_FLAG_SEPARATE_ROUTE])
@pytest.mark.parametrize("name", list(CASES))
def test_f16_roundtrip(name, flags):
    harness.roundtrip(CASES[name], seed=3, flags=flags)


def test_f16_outputs_are_float16_tensors():
    import torch
    wl = CASES["c1_mode0"]
    inp = workloads.generate(wl, seed=0)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    assert dev_in["x"].dtype == torch.float16 and out["expand_x"].dtype == torch.float16
    with pytest.raises(TypeError):                     # a bf16 x under an fp16 config
        cq.dispatch(cfg, dev_in["x"].view(torch.bfloat16), dev_in["ids"])


@pytest.mark.parametrize("name", ["c1_mode2", "int8_h7168", "mx_clip_fp4_special",
                                  "elementwise_h1030"])
def test_f16_int8_block_combine(name):
    import torch
    wl = CASES[name]
    inp = workloads.generate(wl, seed=1)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    rng = np.random.default_rng(21)
    v = rng.standard_normal((wl.cap, wl.H), dtype=np.float32)
    v *= rng.choice(np.float32([1e-4, 1.0, 300.0]), (wl.cap, 1))
    eo = workloads.f32_to_f16_bits(v)
    codes_ref, sc_ref = oracle.combine_quantize(ocfg, eo, ref["recv_offsets"])
    y_ref = oracle.combine_int8(ocfg, codes_ref, sc_ref, inp["expert_ids"], ref["expand_idx"],
                                inp["expert_scales"], ref["ep_recv_count"],
                                ref["recv_offsets"], mask=inp.get("mask"), ori_x=inp["x"])
    codes, scales = cq.combine_quantize(cfg, harness.tok_dev(eo, 1), out["recv_offsets"])
    y = cq.combine_int8(cfg, codes, scales, dev_in["ids"], out["expand_idx"],
                        harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                        out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    P = int(ref["recv_offsets"][-1])
    np.testing.assert_array_equal(harness.host(codes)[:P], codes_ref[:P], err_msg="codes")
    np.testing.assert_array_equal(harness.host(scales)[:P].view(np.uint32),
                                  sc_ref[:P].view(np.uint32), err_msg="block scales")
    harness.check_combine_tolerance(harness.host(y), y_ref, token_dtype=1)


@pytest.mark.parametrize("name", ["c1_mode2", "mx_clip_fp4_special", "elementwise_h1030"])
def test_f16_scatter_back_with_shared(name):
    import torch
    wl = CASES[name]
    inp = workloads.generate(wl, seed=2)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg = harness.lib_cfg(wl)
    x = harness.tok_dev(inp["x"], 1)
    ids = harness.to_dev(inp["expert_ids"])
    mask = harness.to_dev(inp.get("mask"))
    w = harness.to_dev(inp["expert_scales"])
    out = cq.dispatch(cfg, x, ids, harness.to_dev(inp.get("scales")), mask, expert_scales=w)
    rng = np.random.default_rng(31)
    eo = workloads.f32_to_f16_bits(rng.standard_normal((wl.cap, wl.H), dtype=np.float32))
    shared = workloads.f32_to_f16_bits(rng.standard_normal((wl.W, wl.BS, wl.H),
                                                           dtype=np.float32))
    y_ref = oracle.combine_scatter(ocfg, eo, ref["assist_info"], ref["recv_offsets"],
                                   inp["expert_ids"], inp["expert_scales"],
                                   mask=inp.get("mask"), ori_x=inp["x"], shared_x=shared)
    y = cq.combine_scatter(cfg, harness.tok_dev(eo, 1), out["assist_info"], out["recv_offsets"],
                           ids, w, mask, x, harness.tok_dev(shared, 1))
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)
    harness.check_combine_tolerance(harness.host(y), y_ref, token_dtype=1)
