"""GPU checks of the launch plans (prepare_*): a plan checks and marshals one C-ABI call
once; each launch enqueues it again with the same tensors.  Outputs must match the CPU oracle
(dispatch bit for bit, combine within 1e-2 relative / 1e-3 absolute) after the inputs are
rewritten in place, on a side stream, and when the launches are captured in a HIP graph and
replayed with new inputs between replays.  Repeated calls of every entry point leave the
device's free memory unchanged (the library allocates nothing)."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload

CASES = {
    "c1_mode2": workloads.C1_MODE2,
    "mx_e5m2_e8m0_mask": WL("mx_e5m2_e8m0_mask", W=4, E=32, BS=60, H=2048, K=8, quant_mode=4,
                            out_dtype=3, scale_format=1, mask_kind=1,
                            inactive_tokens_per_rank=6, copy_expert_num=1),
    # per-expert scales past the pick kernel's limit (17,408 picks: windows of tokens)
    "smooth_windows": WL("plan_smooth_windows", W=8, E=32, BS=272, H=2048, K=8, quant_mode=2,
                         scales_kind=3, zero_expert_num=1),
}


def _expect(wl, inp, eo):
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    y_ref = oracle.combine(ocfg, eo, inp["expert_ids"], ref["expand_idx"],
                           inp["expert_scales"], ref["ep_recv_count"], ref["recv_offsets"],
                           mask=inp.get("mask"), ori_x=inp["x"])
    return ref, y_ref


def _plans(wl, inp, eo_dev):
    import combine_quant_amd as cq
    cfg = harness.lib_cfg(wl)
    x = harness.bf16_dev(inp["x"])
    ids = harness.to_dev(inp["expert_ids"])
    mask = harness.to_dev(inp.get("mask"))
    sm = harness.to_dev(inp.get("scales"))
    w = harness.to_dev(inp["expert_scales"])
    d, out = cq.prepare_dispatch(cfg, x, ids, sm, mask)
    c, y = cq.prepare_combine(cfg, eo_dev, ids, out["expand_idx"], w, out["ep_recv_count"],
                              out["recv_offsets"], mask, x)
    return dict(x=x, ids=ids, mask=mask, scales=sm, w=w), d, out, c, y


def _refill(dev_in, inp):
    import torch
    dev_in["x"].copy_(harness.bf16_dev(inp["x"]))
    dev_in["ids"].copy_(harness.to_dev(inp["expert_ids"]))
    if dev_in["mask"] is not None:
        dev_in["mask"].copy_(harness.to_dev(inp["mask"]))
    if dev_in["scales"] is not None:
        dev_in["scales"].copy_(harness.to_dev(inp["scales"]))
    dev_in["w"].copy_(harness.to_dev(inp["expert_scales"]))
    torch.cuda.synchronize()


def _eo(wl, seed):
    rng = np.random.default_rng(seed)
    return workloads.f32_to_bf16_bits(rng.standard_normal((wl.cap, wl.H), dtype=np.float32))


@pytest.mark.parametrize("name", list(CASES))
def test_plan_relaunch_with_new_inputs(name):
    import torch
    wl = CASES[name]
    eo = _eo(wl, 9)
    eo_dev = harness.bf16_dev(eo)
    inp0 = workloads.generate(wl, seed=0)
    dev_in, d, out, c, y = _plans(wl, inp0, eo_dev)
    side = torch.cuda.Stream()
    for seed, stream in ((0, None), (1, None), (2, side)):
        inp = workloads.generate(wl, seed=seed)
        _refill(dev_in, inp)
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        d(stream)
        c(stream)
        torch.cuda.synchronize()
        ref, y_ref = _expect(wl, inp, eo)
        harness.compare_dispatch(wl, inp, out, ref)
        harness.check_combine_tolerance(harness.host(y), y_ref)


def test_plans_captured_in_a_graph():
    """Capture dispatch + combine plan launches once; replay after rewriting the inputs in
    place, with eager work and synchronizations between replays; every replay must match the
    oracle on its own inputs."""
    import torch
    wl = CASES["mx_e5m2_e8m0_mask"]
    eo = _eo(wl, 4)
    eo_dev = harness.bf16_dev(eo)
    dev_in, d, out, c, y = _plans(wl, workloads.generate(wl, seed=0), eo_dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm up on the capture stream
        d()
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        d()
        c()
    for seed in (5, 6, 7):
        inp = workloads.generate(wl, seed=seed)
        _refill(dev_in, inp)
        g.replay()
        torch.cuda.synchronize()
        ref, y_ref = _expect(wl, inp, eo)
        harness.compare_dispatch(wl, inp, out, ref)
        harness.check_combine_tolerance(harness.host(y), y_ref)
        torch.zeros(1024, device="cuda").sum().item()     # eager work between replays


def test_library_calls_allocate_no_device_memory():
    """The C ABI never allocates: with every buffer made up front, repeated calls of each
    entry point leave the device's free memory unchanged."""
    import torch
    import combine_quant_amd as cq
    wl = CASES["mx_e5m2_e8m0_mask"]
    inp = workloads.generate(wl, seed=1)
    eo_dev = harness.bf16_dev(_eo(wl, 2))
    dev_in, d, out, c, y = _plans(wl, inp, eo_dev)
    cfg = harness.lib_cfg(wl)
    q, (codes, bscales) = cq.prepare_combine_quantize(cfg, eo_dev, out["recv_offsets"])
    c8, _ = cq.prepare_combine_int8(cfg, codes, bscales, dev_in["ids"], out["expand_idx"],
                                    dev_in["w"], out["ep_recv_count"], out["recv_offsets"],
                                    dev_in["mask"], dev_in["x"])
    ys, _ = cq.prepare_combine_scatter(cfg, eo_dev, out["assist_info"], out["recv_offsets"],
                                       dev_in["ids"], dev_in["w"], dev_in["mask"], dev_in["x"])
    calls = (d, c, q, c8, ys)
    for f in calls:                      # first calls load the code objects
        f()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(20):
        for f in calls:
            f()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
