"""GPU: dispatch writes nothing past its routed rows.

Every row-indexed output (expand_x, dynamic_scales, assist_info, expand_scales) is allocated with
spare rows past W*BS*K and filled with a sentinel byte before the call; afterwards rows
[recv_offsets[W], capacity) must still hold the sentinel in every byte, and rows below it must
match the oracle.  The cases cover each scatter kernel: window workgroups with per-expert
scales on rows that end inside a wave's slots (their loads and stores go through range-checked
buffer resources), windows that span source ranks, MX rows with a pad scale, E2M1 pairs and
reciprocal scales, masks and special experts (fewer routed rows than picks), one workgroup per
pick, routing inside the scatter launch, and the element-wise kernel."""
import numpy as np
import pytest

import harness
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload
SENTINEL = 0xA5
SPARE_ROWS = 3

CASES = {
    "tile_per_expert_token_ragged": WL("guard_tile_token", W=4, E=32, BS=512, H=1056, K=16,
                                       quant_mode=2, scales_kind=3),
    "tile_per_expert_group_masked": WL("guard_tile_group", W=4, E=32, BS=512, H=1160, K=16,
                                       quant_mode=3, out_dtype=2, scales_kind=3, mask_kind=2,
                                       inactive_tokens_per_rank=9),
    "window_spans_ranks_masked": WL("guard_window", W=100, E=200, BS=23, H=1096, K=8,
                                    quant_mode=2, scales_kind=3, mask_kind=2,
                                    inactive_tokens_per_rank=3, zero_expert_num=1,
                                    copy_expert_num=1),
    "mx_fp4_recip_special": WL("guard_mx_fp4", W=4, E=64, BS=70, H=2064, K=16, quant_mode=5,
                               out_dtype=4, scale_format=2, zero_expert_num=2,
                               copy_expert_num=2, mask_kind=2, inactive_tokens_per_rank=7),
    "mx_e8m0_pad": WL("guard_mx_e8m0", W=4, E=32, BS=60, H=1056, K=6, quant_mode=4,
                      scale_format=1),
    "pick_kernel_e5m2_masked": WL("guard_pick", W=8, E=64, BS=65, H=7168, K=8, quant_mode=2,
                                  out_dtype=3, scales_kind=3, mask_kind=2,
                                  inactive_tokens_per_rank=5),
    "fused_small_mode2": WL("guard_fused", W=2, E=8, BS=16, H=1024, K=2, quant_mode=2,
                            zero_expert_num=1, mask_kind=1, inactive_tokens_per_rank=3),
    "element_wise_h1030": WL("guard_elem", W=2, E=8, BS=33, H=1030, K=3, quant_mode=5,
                             out_dtype=3, scale_format=1),
}


def _bytes(t):
    import torch
    return t.contiguous().view(torch.uint8).view(t.shape[0], -1)


@pytest.mark.parametrize("name", list(CASES))
def test_nothing_written_past_the_routed_rows(name):
    import torch
    import combine_quant_amd as cq
    wl = CASES[name]
    inp = workloads.generate(wl, seed=5)
    _, ref = harness.oracle_dispatch(wl, inp)
    cap = wl.W * wl.BS * wl.K + SPARE_ROWS
    cfg = harness.lib_cfg(wl, cap=cap)
    out = cq.alloc_dispatch_outputs(cfg)
    out["expand_scales"] = torch.empty((cap,), dtype=torch.float32, device="cuda")
    guarded = ["expand_x", "assist_info", "expand_scales"]
    if out["dynamic_scales"] is not None:
        guarded.append("dynamic_scales")
    for k in guarded:
        _bytes(out[k]).fill_(SENTINEL)
    x = harness.tok_dev(inp["x"], wl.token_dtype)
    ids = harness.to_dev(inp["expert_ids"])
    sm = harness.to_dev(inp.get("scales"))
    mask = harness.to_dev(inp.get("mask"))
    w = harness.to_dev(inp["expert_scales"])
    o = cq.dispatch(cfg, x, ids, sm, mask, out=out, expert_scales=w)
    torch.cuda.synchronize()
    P = int(o["recv_offsets"][-1].item())
    assert P <= wl.W * wl.BS * wl.K
    for k in guarded:
        tail = _bytes(o[k])[P:]
        assert tail.shape[0] == cap - P
        bad = int((tail != SENTINEL).sum().item())
        assert bad == 0, f"{k}: {bad} bytes written past row {P}"
    harness.compare_dispatch(wl, inp, {k: v for k, v in o.items() if k != "expand_scales"}, ref)
    # each routed row's weight is its pick's
    ai = harness.host(o["assist_info"])[:P].astype(np.int64)
    want = inp["expert_scales"][ai[:, 0], ai[:, 1], ai[:, 2]]
    np.testing.assert_array_equal(harness.host(o["expand_scales"])[:P].view(np.uint32),
                                  np.ascontiguousarray(want, np.float32).view(np.uint32))
