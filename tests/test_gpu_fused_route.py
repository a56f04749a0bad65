"""GPU parity of the small-batch dispatch, which routes inside the scatter launch.

For W*BS*K <= 2048 picks and E*W <= 4096 (vectorised path) moe_dispatch computes the
counts, prefix sums and expand_idx in the scatter workgroups; MOE_DC_FLAG_SEPARATE_ROUTE
forces the route and scan kernels.  Every case runs both ways: each is compared with the CPU
oracle bit for bit, and the two with each other.  The fused launch never touches the
workspace (the separate route and scan keep their counts there), which shows which path ran.
Cases cover masks of both kinds, zero/copy experts, duplicate picks inside a token, both
expert_token_nums types, every scales shape, fp4 codes and both limits exactly."""
import numpy as np
import pytest

import harness
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload

CASES = {
    "c1_mode0": workloads.C1_MODE0,
    "c1_mode2": workloads.C1_MODE2,
    "randint_dups_mask2_special": WL("randint_dups_mask2_special", W=4, E=16, BS=40, H=1024,
                                     K=8, quant_mode=2, routing="randint", mask_kind=2,
                                     inactive_tokens_per_rank=5, zero_expert_num=1,
                                     copy_expert_num=1),
    "mask1_etn0_mx": WL("mask1_etn0_mx", W=8, E=64, BS=16, H=2048, K=6, quant_mode=4,
                        mask_kind=1, inactive_tokens_per_rank=3, expert_token_nums_type=0),
    "per_expert_group_e4m3": WL("per_expert_group_e4m3", W=2, E=8, BS=64, H=1152, K=4,
                                quant_mode=3, scales_kind=3, out_dtype=2),
    "sample_bs8_mx_e5m2_e8m0": WL("sample_bs8_mx_e5m2_e8m0", W=8, E=32, BS=8, H=7168, K=8,
                                  quant_mode=4, out_dtype=3, scale_format=1),
    "picks_at_limit": WL("picks_at_limit", W=2, E=32, BS=128, H=1024, K=8, quant_mode=2),
    "counts_at_limit_fp4": WL("counts_at_limit_fp4", W=4, E=1024, BS=8, H=1040, K=16,
                              quant_mode=5, out_dtype=4, scale_format=1),
    "one_token_per_rank": WL("one_token_per_rank", W=16, E=256, BS=1, H=7168, K=8,
                             quant_mode=2),
    "smooth_per_expert_int8": WL("smooth_per_expert_int8", W=8, E=64, BS=16, H=7168, K=8,
                                 quant_mode=2, scales_kind=3, outlier_prob=0.01),
    "static_shared_row": WL("static_shared_row", W=4, E=32, BS=16, H=2048, K=6, quant_mode=1,
                            scales_kind=2),
    "mx_e2m1_fp32_ragged": WL("mx_e2m1_fp32_ragged", W=4, E=16, BS=32, H=2064, K=4,
                              quant_mode=4, out_dtype=4),
    "mxclip_e4m3_recip": WL("mxclip_e4m3_recip", W=8, E=32, BS=8, H=7200, K=8, quant_mode=5,
                            scale_format=2, mask_kind=1, inactive_tokens_per_rank=2),
}
# just past the limits: the separate kernels run whatever the flag says
PAST_LIMIT = {
    "picks_past_limit": WL("picks_past_limit", W=2, E=32, BS=129, H=1024, K=8, quant_mode=2),
    "counts_past_limit": WL("counts_past_limit", W=8, E=1024, BS=4, H=1024, K=8,
                            quant_mode=2),
}

SENTINEL = 0xA5


def _run(wl, inp, flags):
    import torch
    import combine_quant_amd as cq
    cfg = harness.lib_cfg(wl, flags=flags)
    out = cq.alloc_dispatch_outputs(cfg)
    for k in ("workspace", "expand_idx", "ep_recv_count", "expert_token_nums", "recv_offsets"):
        out[k].view(torch.uint8).fill_(SENTINEL)
    x = harness.bf16_dev(inp["x"])
    ids = harness.to_dev(inp["expert_ids"])
    sm = harness.to_dev(inp.get("scales"))
    mask = harness.to_dev(inp.get("mask"))
    w = harness.to_dev(inp["expert_scales"])
    cq.dispatch(cfg, x, ids, sm, mask, out=out, expert_scales=w)
    torch.cuda.synchronize()
    return out


def _check_both_ways(wl, seed, expect_fused):
    import combine_quant_amd as cq
    inp = workloads.generate(wl, seed=seed)
    _, ref = harness.oracle_dispatch(wl, inp)
    P = int(ref["recv_offsets"][-1])
    got = []
    for flags in (0, cq.MOE_DC_FLAG_SEPARATE_ROUTE):
        out = _run(wl, inp, flags)
        o = harness.compare_dispatch(wl, inp, out, ref)
        ws = harness.host(out["workspace"])
        untouched = bool((ws == SENTINEL).all())
        assert untouched == (expect_fused and flags == 0), (flags, untouched)
        # each routed row carries its pick's weight
        s_, i_, k_ = ref["assist_info"][:P].T
        np.testing.assert_array_equal(harness.host(out["expand_scales"])[:P],
                                      inp["expert_scales"][s_, i_, k_])
        got.append(o)
    for k in ("expand_x", "assist_info"):
        np.testing.assert_array_equal(got[0][k][:P], got[1][k][:P], err_msg=k)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("seed", [0, 3])
def test_fused_route_matches_the_oracle_and_the_separate_kernels(name, seed):
    _check_both_ways(CASES[name], seed, expect_fused=True)


@pytest.mark.parametrize("name", list(PAST_LIMIT))
def test_past_the_limits_the_separate_kernels_run(name):
    _check_both_ways(PAST_LIMIT[name], 1, expect_fused=False)


def test_fused_roundtrip_combine():
    assert harness.roundtrip(workloads.C1_MODE2, seed=7) >= 0
