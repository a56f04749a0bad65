"""Independent calls on different streams: the library keeps no device state of its own
between calls (every scratch word lives in the caller's workspace), so dispatch -> combine
round trips of different configurations, each on its own stream with its own buffers, can
run at the same time.  Their launches are interleaved across four streams and every
result must match the CPU oracle exactly as it does alone (dispatch bit for bit, combine
within 1e-2 relative / 1e-3 absolute)."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

# one small batch that routes inside the scatter launch, and three that use the route and
# scan kernels (per-expert scales through one workgroup per pick, and through windows of tokens;
# MX with special experts and a per-pick mask)
CASES = [
    workloads.Workload("streams_small", W=4, E=16, BS=24, H=1024, K=4, quant_mode=2),
    workloads.Workload("streams_smooth", W=4, E=32, BS=160, H=2048, K=8, quant_mode=2,
                       scales_kind=3),
    workloads.Workload("streams_smooth_windows", W=8, E=32, BS=272, H=1056, K=8, quant_mode=2,
                       scales_kind=3, mask_kind=1, inactive_tokens_per_rank=11),
    workloads.Workload("streams_mx", W=8, E=32, BS=96, H=1024, K=6, quant_mode=5,
                       zero_expert_num=1, copy_expert_num=1, mask_kind=2,
                       inactive_tokens_per_rank=8, routing="randint"),
]


def test_round_trips_on_several_streams_at_once():
    import torch
    import combine_quant_amd as cq
    dev = torch.device("cuda")
    jobs = []
    for n, wl in enumerate(CASES):
        inp = workloads.generate(wl, seed=40 + n)
        cfg = harness.lib_cfg(wl)
        rng = np.random.default_rng(90 + n)
        eo = workloads.f32_to_bf16_bits(rng.standard_normal((wl.cap, wl.H), dtype=np.float32))
        jobs.append(dict(
            wl=wl, inp=inp, cfg=cfg, eo_host=eo,
            x=harness.bf16_dev(inp["x"]), ids=harness.to_dev(inp["expert_ids"]),
            scales=harness.to_dev(inp.get("scales")), mask=harness.to_dev(inp.get("mask")),
            w=harness.to_dev(inp["expert_scales"]), eo=harness.bf16_dev(eo),
            out=cq.alloc_dispatch_outputs(cfg, dev),
            y=torch.empty((wl.W, wl.BS, wl.H), dtype=torch.bfloat16, device=dev),
            stream=torch.cuda.Stream()))
    torch.cuda.synchronize()          # every buffer is ready before the side streams start

    # dispatches first on all the streams, then the combines, so the kernels of different
    # calls are in flight together
    for j in jobs:
        cq.dispatch(j["cfg"], j["x"], j["ids"], j["scales"], j["mask"], out=j["out"],
                    stream=j["stream"])
    for j in jobs:
        o = j["out"]
        cq.combine(j["cfg"], j["eo"], j["ids"], o["expand_idx"], j["w"], o["ep_recv_count"],
                   o["recv_offsets"], j["mask"], j["x"], j["y"], stream=j["stream"])
    torch.cuda.synchronize()

    for j in jobs:
        wl, inp = j["wl"], j["inp"]
        ocfg, ref = harness.oracle_dispatch(wl, inp)
        harness.compare_dispatch(wl, inp, j["out"], ref)
        y_ref = oracle.combine(ocfg, j["eo_host"], inp["expert_ids"], ref["expand_idx"],
                               inp["expert_scales"], ref["ep_recv_count"],
                               ref["recv_offsets"], mask=inp.get("mask"), ori_x=inp["x"])
        harness.check_combine_tolerance(harness.host(j["y"]), y_ref)
