"""The library enqueues kernels only (no allocation, memset or host synchronization), so a
whole dispatch -> combine round trip can be captured into a HIP graph and replayed.  Each
replay runs on new input contents written into the captured buffers, with eager work and
synchronizations between replays, and every output of every replay must equal the eager
result on the same inputs bit for bit."""
import numpy as np
import pytest

import harness
import workloads

pytestmark = pytest.mark.gpu

CASES = {
    "int8_masked_special": workloads.Workload(
        "graph_int8", W=4, E=32, BS=60, H=1024, K=8, quant_mode=2, zero_expert_num=1,
        copy_expert_num=1, mask_kind=2, inactive_tokens_per_rank=6, routing="randint"),
    "mx_e5m2_e8m0": workloads.Workload("graph_mx", W=4, E=32, BS=40, H=2048, K=6,
                                       quant_mode=5, out_dtype=3, scale_format=1),
    # 6,400 picks: routing and prefix sums run as kernels of their own (the two cases above
    # route inside the scatter launch)
    "int8_three_launches": workloads.Workload("graph_int8_large", W=4, E=32, BS=200, H=1024,
                                              K=8, quant_mode=2, mask_kind=1,
                                              inactive_tokens_per_rank=9),
    # per-expert scales: 3,200 picks (one workgroup per pick) and 17,408 picks (one workgroup
    # per window of tokens and expert)
    "smooth_pick_kernel": workloads.Workload("graph_smooth_pick", W=4, E=32, BS=100, H=2048,
                                             K=8, quant_mode=2, scales_kind=3, mask_kind=2,
                                             inactive_tokens_per_rank=5),
    "smooth_window_kernel": workloads.Workload("graph_smooth_window", W=8, E=32, BS=272,
                                               H=1024, K=8, quant_mode=3, out_dtype=2,
                                               scales_kind=3),
}


def _outputs(out, y):
    d = {k: v for k, v in out.items() if v is not None and k != "workspace"}
    d["y"] = y
    return d


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    import torch
    import combine_quant_amd as cq
    wl = CASES[name]
    cfg = harness.lib_cfg(wl)
    dev = torch.device("cuda")
    draws = [workloads.generate(wl, seed=s) for s in range(4)]
    rng = np.random.default_rng(0)
    eos = [workloads.f32_to_bf16_bits(rng.standard_normal((wl.cap, wl.H)).astype(np.float32))
           for _ in range(4)]

    def load(inp, eo):
        return dict(x=harness.bf16_dev(inp["x"]), ids=harness.to_dev(inp["expert_ids"]),
                    scales=harness.to_dev(inp.get("scales")), mask=harness.to_dev(inp.get("mask")),
                    w=harness.to_dev(inp["expert_scales"]), eo=harness.bf16_dev(eo))

    def run(t, out, y, stream=None):
        cq.dispatch(cfg, t["x"], t["ids"], t["scales"], t["mask"], out=out, stream=stream)
        cq.combine(cfg, t["eo"], t["ids"], out["expand_idx"], t["w"], out["ep_recv_count"],
                   out["recv_offsets"], t["mask"], t["x"], y, stream=stream)

    static = load(draws[0], eos[0])
    g_out = cq.alloc_dispatch_outputs(cfg, dev)
    g_y = torch.empty((wl.W, wl.BS, wl.H), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm-up outside the capture
        run(static, g_out, g_y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(static, g_out, g_y)
    torch.cuda.synchronize()

    for rep in range(1, 4):
        fresh = load(draws[rep], eos[rep])
        for k, v in fresh.items():
            if v is not None:
                static[k].copy_(v)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_out = cq.alloc_dispatch_outputs(cfg, dev)
        e_y = torch.empty_like(g_y)
        run(fresh, e_out, e_y)                          # eager, on the same input contents
        torch.cuda.synchronize()
        got, want = _outputs(g_out, g_y), _outputs(e_out, e_y)
        P = int(want["recv_offsets"][-1].item())
        for k in want:
            a, b = got[k], want[k]
            if k in ("expand_x", "dynamic_scales", "assist_info"):
                a, b = a[:P], b[:P]
            assert torch.equal(a.view(torch.uint8) if a.dtype.itemsize == 1 else a,
                               b.view(torch.uint8) if b.dtype.itemsize == 1 else b), (rep, k)
