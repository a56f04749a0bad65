"""Test harness: runs the same seeded inputs through the HIP library and the CPU oracle.

The GPU side only ever calls the C ABI through combine_quant_amd's binding; the oracle side
only ever calls oracle/.  The two meet here, in the comparisons.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def oracle_cfg(wl: workloads.Workload, etn_type=None):
    return oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, quant_mode=wl.quant_mode,
                           zero_expert_num=wl.zero_expert_num,
                           copy_expert_num=wl.copy_expert_num,
                           expert_token_nums_type=wl.expert_token_nums_type if etn_type is None
                           else etn_type,
                           mask_kind=wl.mask_kind, out_dtype=wl.out_dtype,
                           scales_kind=wl.scales_kind, scale_format=wl.scale_format,
                           token_dtype=wl.token_dtype)


def lib_cfg(wl: workloads.Workload, cap=None, flags=0):
    import combine_quant_amd as cq
    return cq.make_config(wl.W, wl.E, wl.BS, wl.H, wl.K, wl.quant_mode,
                          zero_expert_num=wl.zero_expert_num,
                          copy_expert_num=wl.copy_expert_num,
                          expert_token_nums_type=wl.expert_token_nums_type,
                          mask_kind=wl.mask_kind, cap=cap, out_dtype=wl.out_dtype,
                          scales_kind=wl.scales_kind, scale_format=wl.scale_format,
                          flags=flags, token_dtype=wl.token_dtype)


def to_dev(a, dtype=None, device="cuda"):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def bf16_dev(a_u16, device="cuda"):
    import torch
    return to_dev(a_u16, torch.bfloat16, device)


def tok_dev(a_u16, token_dtype=0, device="cuda"):
    """Token bit patterns as a device tensor: bfloat16, or float16 for token_dtype 1."""
    import torch
    return to_dev(a_u16, torch.float16 if token_dtype == 1 else torch.bfloat16, device)


def host(t):
    import torch
    if t is None:
        return None
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        t = t.view(torch.uint8)
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 and t.dtype == torch.int16 else a


def gpu_dispatch(wl, inp, cfg=None, device="cuda"):
    import combine_quant_amd as cq
    cfg = lib_cfg(wl) if cfg is None else cfg
    x = tok_dev(inp["x"], wl.token_dtype, device)
    ids = to_dev(inp["expert_ids"], device=device)
    sm = to_dev(inp.get("scales"), device=device)
    mask = to_dev(inp.get("mask"), device=device)
    out = cq.dispatch(cfg, x, ids, sm, mask)
    return cfg, dict(x=x, ids=ids, mask=mask), out


def compare_dispatch(wl, inp, out_dev, ref, rows=None):
    """Bit-exact comparison of every dispatch output (rows: optional subset of rows to
    compare for the per-row payload; default every routed row)."""
    o = {k: host(v) for k, v in out_dev.items() if k != "workspace"}
    np.testing.assert_array_equal(o["expand_idx"], ref["expand_idx"], err_msg="expand_idx")
    np.testing.assert_array_equal(o["ep_recv_count"], ref["ep_recv_count"],
                                  err_msg="ep_recv_count")
    np.testing.assert_array_equal(o["expert_token_nums"], ref["expert_token_nums"],
                                  err_msg="expert_token_nums")
    np.testing.assert_array_equal(o["recv_offsets"], ref["recv_offsets"],
                                  err_msg="recv_offsets")
    P = int(ref["recv_offsets"][-1])
    sel = slice(0, P) if rows is None else np.asarray(rows)
    np.testing.assert_array_equal(o["assist_info"][sel], ref["assist_info"][sel],
                                  err_msg="assist_info")
    ex = o["expand_x"][sel]
    rex = ref["expand_x"][sel]
    np.testing.assert_array_equal(ex.view(np.uint8), rex.view(np.uint8), err_msg="expand_x")
    if "dynamic_scales" in ref:
        a, b = o["dynamic_scales"][sel], ref["dynamic_scales"][sel]
        assert a.dtype == b.dtype and a.shape == b.shape, (a.dtype, b.dtype, a.shape, b.shape)
        np.testing.assert_array_equal(np.ascontiguousarray(a).view(np.uint8),
                                      np.ascontiguousarray(b).view(np.uint8),
                                      err_msg="dynamic_scales")
    else:
        assert o.get("dynamic_scales") is None
    return o


def check_combine_tolerance(y_gpu_u16, y_ref_u16, rtol=1e-2, atol=1e-3, token_dtype=0):
    a = workloads.tok_bits_to_f32(y_gpu_u16, token_dtype).astype(np.float64)
    b = workloads.tok_bits_to_f32(y_ref_u16, token_dtype).astype(np.float64)
    bad = np.abs(a - b) > atol + rtol * np.abs(b)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} elements out of tolerance"
    return int((y_gpu_u16 != y_ref_u16).sum())


def oracle_dispatch(wl, inp, etn_type=None):
    cfg = oracle_cfg(wl, etn_type)
    return cfg, oracle.dispatch(cfg, inp["x"], inp["expert_ids"], scales=inp.get("scales"),
                                mask=inp.get("mask"))


def roundtrip(wl, seed=0, flags=0):
    """Dispatch compared bit for bit, then combine over random expert outputs (of the
    workload's token type) compared within tolerance; returns the number of elements that
    differ at all."""
    import torch
    import combine_quant_amd as cq
    inp = workloads.generate(wl, seed=seed)
    ocfg, ref = oracle_dispatch(wl, inp)
    cfg, dev_in, out = gpu_dispatch(wl, inp, cfg=lib_cfg(wl, flags=flags))
    torch.cuda.synchronize()
    compare_dispatch(wl, inp, out, ref)
    rng = np.random.default_rng(seed + 77)
    eo = workloads.f32_to_tok_bits(rng.standard_normal((wl.cap, wl.H), dtype=np.float32),
                                   wl.token_dtype)
    y_ref = oracle.combine(ocfg, eo, inp["expert_ids"], ref["expand_idx"],
                           inp["expert_scales"], ref["ep_recv_count"], ref["recv_offsets"],
                           mask=inp.get("mask"), ori_x=inp["x"])
    y = cq.combine(cfg, tok_dev(eo, wl.token_dtype), dev_in["ids"], out["expand_idx"],
                   to_dev(inp["expert_scales"]), out["ep_recv_count"],
                   out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    return check_combine_tolerance(host(y), y_ref, token_dtype=wl.token_dtype)
