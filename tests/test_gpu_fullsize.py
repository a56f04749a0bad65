"""GPU parity at the full workload sizes, in the library's normal launch configuration.

Every output is compared in full against the oracle run over the whole workload: the routing
outputs, every routed row of expand_x, dynamic_scales and assist_info bit for bit, and every
element of the combine output y within 1e-2 relative / 1e-3 absolute (the number of elements
that are bit-identical is printed and asserted to be all of them).
"""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

FULL = ["c3_w16_mxfp8_zipf", "c4_w16_int8_roundtrip", "c5_w32_mxclip_special"]


def _check_y(tag, y_dev, y_ref, token_dtype=0):
    y = harness.host(y_dev)
    ndiff = harness.check_combine_tolerance(y.reshape(y_ref.shape), y_ref,
                                            token_dtype=token_dtype)
    print(f"[{tag}] y: {y_ref.size - ndiff} of {y_ref.size} elements bit-identical",
          flush=True)
    assert ndiff == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_fullsize_dispatch_and_combine(name):
    import torch
    import combine_quant_amd as cq
    wl = workloads.WORKLOADS[name]
    inp = workloads.generate(wl, seed=0)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)        # every routed row, bit for bit
    P = int(ref["recv_offsets"][-1])
    print(f"[{name}] dispatch: {P} routed rows identical", flush=True)
    del ref["expand_x"]

    # combine on bf16 N(0,1) expert outputs drawn on the device, one per packed row; the
    # oracle reads the host copy of the same bytes
    eo = workloads.expert_out_torch(wl, wl.cap, seed=0)
    y = cq.combine(cfg, eo, dev_in["ids"], out["expand_idx"],
                   harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                   out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    eo_h = harness.host(eo)
    del eo
    y_ref = oracle.combine(ocfg, eo_h, inp["expert_ids"], ref["expand_idx"],
                           inp["expert_scales"], ref["ep_recv_count"], ref["recv_offsets"],
                           mask=inp.get("mask"), ori_x=inp["x"])
    _check_y(name, y, y_ref)


@pytest.mark.timeout(600)
def test_c4_identity_dequant_roundtrip_fullsize():
    """Full dispatch (int8) -> identity-dequant expert (bf16(q*scale)) -> combine, at full
    size: every output element against the oracle's own round trip, and every token against
    the fp32 weighted sum of x within the int8 quantization bound."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C4
    inp = workloads.generate(wl, seed=0)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo = (out["expand_x"].float() * out["dynamic_scales"][:, None]).to(torch.bfloat16)
    w_dev = harness.to_dev(inp["expert_scales"])
    y = cq.combine(cfg, eo, dev_in["ids"], out["expand_idx"], w_dev, out["ep_recv_count"],
                   out["recv_offsets"])
    # property at any size: y ~ sum_k w_k x within half an int8 step + bf16 roundings
    xf = dev_in["x"].float()
    wsum = w_dev.sum(dim=2, keepdim=True)
    amax = xf.abs().amax(dim=2, keepdim=True)
    err = (y.float() - wsum * xf).abs()
    bound = 0.5 * amax / 127 + xf.abs() * 2.0 ** -7 + amax * 2.0 ** -8
    assert bool((err <= bound).all())
    torch.cuda.synchronize()
    # the oracle's round trip: its own codes and scales, dequantized by the same identity
    # expert (one fp32 multiply, bf16 rounding), then its combine
    P = int(ref["recv_offsets"][-1])
    eo_h = np.zeros((wl.cap, wl.H), np.uint16)
    eo_h[:P] = workloads.f32_to_bf16_bits(ref["expand_x"][:P].astype(np.float32) *
                                          ref["dynamic_scales"][:P, None])
    y_ref = oracle.combine(ocfg, eo_h, inp["expert_ids"], ref["expand_idx"],
                           inp["expert_scales"], ref["ep_recv_count"], ref["recv_offsets"])
    _check_y("c4 identity round trip", y, y_ref)
