"""moe_dispatch_no_workspace: moe_dispatch for callers that cannot allocate device memory.

On the GPU, calls in a row (a W=16, H=7168 batch, then a smaller masked MX batch with a
different routing, so the second call runs over the first one's leftovers in the shared
scratch, then a batch with per-expert scales that takes the window kernel) must give exactly
the bytes moe_dispatch gives with a workspace of its own, and
repeated calls must leave the device's free memory unchanged.  On the host, the configs the
1 MiB scratch cannot hold and the id check are refused before any device work.
"""
import ctypes

import numpy as np
import pytest

import harness
import workloads

SMALL = workloads.Workload(name="no_alloc_small", W=8, E=64, BS=128, H=2048, K=8,
                           quant_mode=4, zero_expert_num=1, copy_expert_num=1, mask_kind=2,
                           inactive_tokens_per_rank=13, routing="uniform",
                           description="a smaller masked MX batch with special experts")
SMOOTH = workloads.Workload(name="no_alloc_smooth", W=8, E=64, BS=272, H=2048, K=8,
                            quant_mode=2, scales_kind=3, routing="zipf",
                            description="per-expert scales past the pick kernel's limit")


def _compare(wl, a, b):
    import torch
    torch.cuda.synchronize()
    P = int(harness.host(a["recv_offsets"])[-1])
    for k in ("expand_idx", "ep_recv_count", "expert_token_nums", "recv_offsets"):
        np.testing.assert_array_equal(harness.host(a[k]), harness.host(b[k]), err_msg=k)
    for k in ("expand_x", "dynamic_scales", "assist_info"):
        if a[k] is None:
            assert b[k] is None
            continue
        x, y = harness.host(a[k][:P]), harness.host(b[k][:P])
        np.testing.assert_array_equal(np.ascontiguousarray(x).view(np.uint8),
                                      np.ascontiguousarray(y).view(np.uint8), err_msg=k)
    return P


def _no_workspace(cfg, dev_in, sm, out):
    import combine_quant_amd as cq
    cq.moe_dispatch_no_workspace(cfg, dev_in["x"], dev_in["ids"], sm, dev_in["mask"],
                                 out["expand_x"], out["dynamic_scales"], out["expand_idx"],
                                 out["assist_info"], out["ep_recv_count"],
                                 out["expert_token_nums"], out["recv_offsets"])


@pytest.mark.gpu
def test_no_workspace_dispatch_matches_dispatch_on_two_calls():
    import torch
    import combine_quant_amd as cq
    for wl in (workloads.C4, SMALL, SMOOTH):         # the second call is the smaller one
        inp = workloads.generate(wl, seed=3)
        cfg, dev_in, ref = harness.gpu_dispatch(wl, inp)
        sm = harness.to_dev(inp.get("scales"))
        out = cq.alloc_dispatch_outputs(cfg)
        for k in ("expand_x", "assist_info"):
            out[k].view(torch.uint8).fill_(0xA5)     # a routed row left unwritten would show
        _no_workspace(cfg, dev_in, sm, out)
        P = _compare(wl, ref, out)
        print(f"[{wl.name}] {P} routed rows identical to moe_dispatch", flush=True)


@pytest.mark.gpu
def test_no_workspace_dispatch_allocates_nothing():
    import torch
    import combine_quant_amd as cq
    wl = workloads.C2
    inp = workloads.generate(wl, seed=4)
    cfg, dev_in, ref = harness.gpu_dispatch(wl, inp)
    sm = harness.to_dev(inp.get("scales"))
    out = cq.alloc_dispatch_outputs(cfg)
    _no_workspace(cfg, dev_in, sm, out)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(20):
        _no_workspace(cfg, dev_in, sm, out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
    _compare(wl, ref, out)


def _raw(lib, cfg):
    p = ctypes.c_void_p(16)                          # never dereferenced: refused on the host
    return lib.moe_dispatch_no_workspace(ctypes.byref(cfg), p, p, None, None, None, p, p, p, p,
                                         p, p, p, None, None)


def test_no_workspace_dispatch_refuses_on_the_host():
    import combine_quant_amd as cq
    lib = cq.load_library()
    big = cq.make_config(768, 768, 4, 1024, 2, 2)    # 2.36 MB of counts: beyond 1 MiB
    assert cq.moe_dc_validate(big) == cq.MOE_OK
    assert cq.moe_dc_dispatch_workspace_bytes(big) > (1 << 20)
    assert _raw(lib, big) == cq.MOE_ERR_WORKSPACE
    assert "static scratch" in cq.moe_dc_last_error()
    checked = cq.make_config(16, 256, 512, 7168, 8, 2, flags=cq.MOE_DC_FLAG_CHECK_IDS)
    assert _raw(lib, checked) == cq.MOE_ERR_INVALID_ARG
    assert "CHECK_IDS" in cq.moe_dc_last_error()
    nulls = cq.make_config(16, 256, 512, 7168, 8, 2)
    assert lib.moe_dispatch_no_workspace(ctypes.byref(nulls), *([None] * 13),
                                         None) == cq.MOE_ERR_INVALID_ARG
