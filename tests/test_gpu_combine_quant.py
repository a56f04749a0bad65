"""GPU parity of the combine-side int8 block quantization: moe_combine_quantize (codes and
block scales of every routed expert-output row, bit for bit against the oracle) and
moe_combine_int8 (y within 1e-2 relative / 1e-3 absolute of the oracle, expected to be
bit-identical), through the C ABI, on the vectorized and element-wise kernels."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload

CASES = {
    "c1": workloads.C1_MODE2,
    "ragged_h1056": WL("cq_ragged", W=4, E=32, BS=70, H=1056, K=6, quant_mode=4,
                       routing="zipf"),
    "special_masked_k16": WL("cq_special", W=4, E=64, BS=40, H=2048, K=16, quant_mode=5,
                             zero_expert_num=2, copy_expert_num=2, mask_kind=2,
                             inactive_tokens_per_rank=5),
    "dup_k8_mask1d": WL("cq_dup", W=2, E=8, BS=65, H=1024, K=8, quant_mode=2,
                        routing="randint", zero_expert_num=1, copy_expert_num=1, mask_kind=1,
                        inactive_tokens_per_rank=9),
    "elem_h1030": WL("cq_h1030", W=2, E=8, BS=33, H=1030, K=3, quant_mode=0,
                     copy_expert_num=1),
    # H % 16 != 0 keeps 8-element lanes; K <= 8 with H % 16 == 0 takes 16-element lanes
    "narrow_h1032_copy": WL("cq_h1032", W=3, E=12, BS=50, H=1032, K=5, quant_mode=2,
                            copy_expert_num=2, zero_expert_num=1, routing="randint"),
    "wide_copy_k4": WL("cq_wide_copy", W=2, E=16, BS=90, H=2048, K=4, quant_mode=2,
                       copy_expert_num=1, zero_expert_num=1, mask_kind=2,
                       inactive_tokens_per_rank=7),
}


def _expert_out(wl, seed, scale_mix=True):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((wl.cap, wl.H), dtype=np.float32)
    if scale_mix:                                   # rows and blocks of very different sizes
        v *= rng.choice(np.float32([1e-20, 1e-3, 1.0, 1e3]), (wl.cap, 1))
        v[:, 8:16] = 0.0                            # one all-zero block per row
    return workloads.f32_to_tok_bits(v, wl.token_dtype)


def _run(wl, seed=0, eo=None):
    import torch
    import combine_quant_amd as cq
    inp = workloads.generate(wl, seed=seed)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo = _expert_out(wl, seed + 5) if eo is None else eo
    codes_ref, sc_ref = oracle.combine_quantize(ocfg, eo, ref["recv_offsets"])
    y_ref = oracle.combine_int8(ocfg, codes_ref, sc_ref, inp["expert_ids"], ref["expand_idx"],
                                inp["expert_scales"], ref["ep_recv_count"],
                                ref["recv_offsets"], mask=inp.get("mask"), ori_x=inp["x"])
    codes, scales = cq.combine_quantize(cfg, harness.tok_dev(eo, wl.token_dtype),
                                        out["recv_offsets"])
    y = cq.combine_int8(cfg, codes, scales, dev_in["ids"], out["expand_idx"],
                        harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                        out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    P = int(ref["recv_offsets"][-1])
    np.testing.assert_array_equal(harness.host(codes)[:P], codes_ref[:P], err_msg="codes")
    np.testing.assert_array_equal(harness.host(scales)[:P].view(np.uint32),
                                  sc_ref[:P].view(np.uint32), err_msg="block scales")
    return harness.check_combine_tolerance(harness.host(y), y_ref, token_dtype=wl.token_dtype)


@pytest.mark.parametrize("name", list(CASES))
def test_combine_int8_roundtrip(name):
    assert _run(CASES[name]) == 0


def test_every_bf16_value_as_an_expert_output_element():
    """All finite bf16 patterns spread over the expert rows, in blocks mixing magnitudes:
    the division, the fp16 rounding and the int8 rounding of every value."""
    wl = WL("cq_sweep", W=2, E=8, BS=32, H=1024, K=2, quant_mode=0)
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[np.isfinite(workloads.bf16_bits_to_f32(b))]
    b = np.random.default_rng(1).permutation(b)
    eo = np.zeros(wl.cap * wl.H, np.uint16)
    eo[:len(b)] = b
    assert len(b) <= eo.size
    assert _run(wl, eo=eo.reshape(wl.cap, wl.H)) == 0


def test_rows_past_the_routed_count_are_not_written():
    import torch
    import combine_quant_amd as cq
    wl = CASES["special_masked_k16"]
    inp = workloads.generate(wl, seed=3)
    cfg, _, out = harness.gpu_dispatch(wl, inp)
    codes = torch.full((wl.cap, wl.H), 77, dtype=torch.int8, device="cuda")
    scales = torch.full((wl.cap, (wl.H + 7) // 8), 5.0, dtype=torch.float32, device="cuda")
    eo = harness.bf16_dev(_expert_out(wl, 2))
    cq.combine_quantize(cfg, eo, out["recv_offsets"], out=(codes, scales))
    torch.cuda.synchronize()
    P = int(out["recv_offsets"][-1].item())
    assert P < wl.cap
    assert (codes[P:] == 77).all() and (scales[P:] == 5.0).all()


def test_unaligned_codes_take_the_element_kernels():
    import torch
    import combine_quant_amd as cq
    wl = CASES["c1"]
    inp = workloads.generate(wl, seed=4)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo = _expert_out(wl, 6)
    codes_ref, sc_ref = oracle.combine_quantize(ocfg, eo, ref["recv_offsets"])
    y_ref = oracle.combine_int8(ocfg, codes_ref, sc_ref, inp["expert_ids"], ref["expand_idx"],
                                inp["expert_scales"], ref["ep_recv_count"],
                                ref["recv_offsets"])
    buf = torch.zeros(wl.cap * wl.H + 1, dtype=torch.int8, device="cuda")
    codes = buf[1:].view(wl.cap, wl.H)
    assert codes.data_ptr() % 8 != 0
    scales = torch.empty((wl.cap, wl.H // 8), dtype=torch.float32, device="cuda")
    cq.combine_quantize(cfg, harness.bf16_dev(eo), out["recv_offsets"], out=(codes, scales))
    y = cq.combine_int8(cfg, codes, scales, dev_in["ids"], out["expand_idx"],
                        harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                        out["recv_offsets"])
    torch.cuda.synchronize()
    P = int(ref["recv_offsets"][-1])
    np.testing.assert_array_equal(harness.host(codes)[:P], codes_ref[:P])
    assert harness.check_combine_tolerance(harness.host(y), y_ref) == 0


def test_full_size_sampled():
    """The W=16, BS=512, H=7168, K=8 shape in the bench's launch configuration: 256 sampled
    rows' codes and scales recomputed by the oracle, and every token's output."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C4
    inp = workloads.generate(wl, seed=0)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo_dev = workloads.expert_out_torch(wl, wl.cap, seed=0)
    codes, scales = cq.combine_quantize(cfg, eo_dev, out["recv_offsets"])
    y = cq.combine_int8(cfg, codes, scales, dev_in["ids"], out["expand_idx"],
                        harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                        out["recv_offsets"])
    torch.cuda.synchronize()
    eo = harness.host(eo_dev)
    codes_h, scales_h, y_h = harness.host(codes), harness.host(scales), harness.host(y)
    rng = np.random.default_rng(0)
    for r in rng.choice(wl.cap, 256, replace=False):
        q, sc = oracle.combine_quant_row(eo[r])
        assert (codes_h[r] == q).all() and (scales_h[r].view(np.uint32) == sc.view(np.uint32)).all()
    # every token: the oracle's int8 combine over the library's own (sample-checked) codes
    ocfg = harness.oracle_cfg(wl)
    y_ref = oracle.combine_int8(ocfg, codes_h, scales_h, inp["expert_ids"],
                                harness.host(out["expand_idx"]), inp["expert_scales"],
                                harness.host(out["ep_recv_count"]),
                                harness.host(out["recv_offsets"]))
    assert harness.check_combine_tolerance(y_h, y_ref) == 0
