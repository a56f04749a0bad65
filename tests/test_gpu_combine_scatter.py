"""GPU parity of the row weights (dispatch's expand_scales, bit for bit) and of the
scatter-back combine (moe_combine_scatter: rows returned by their assist_info triples, the
per-token K-sum, the shared expert's output added last) against the CPU oracle, through the
C ABI; combine within 1e-2 relative / 1e-3 absolute, expected bit-identical."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload

CASES = {
    "c1": workloads.C1_MODE2,
    "ragged_k6": WL("sb_ragged", W=4, E=32, BS=70, H=1056, K=6, quant_mode=4, routing="zipf"),
    "special_masked_k16": WL("sb_special", W=4, E=64, BS=40, H=2048, K=16, quant_mode=5,
                             zero_expert_num=2, copy_expert_num=2, mask_kind=2,
                             inactive_tokens_per_rank=5),
    "dup_mask1d": WL("sb_dup", W=2, E=8, BS=65, H=1024, K=8, quant_mode=2, routing="randint",
                     zero_expert_num=1, copy_expert_num=1, mask_kind=1,
                     inactive_tokens_per_rank=9),
    "elem_h1030": WL("sb_h1030", W=2, E=8, BS=33, H=1030, K=3, quant_mode=0,
                     copy_expert_num=1),
}


def _shared(wl, seed):
    return workloads.f32_to_tok_bits(np.random.default_rng(seed).standard_normal(
        (wl.W, wl.BS, wl.H)).astype(np.float32), wl.token_dtype)


def _run(wl, seed, with_shared, workspace=None):
    import torch
    import combine_quant_amd as cq
    inp = workloads.generate(wl, seed=seed)
    ocfg, ref = harness.oracle_dispatch(wl, inp)
    cfg = harness.lib_cfg(wl)
    tok = wl.token_dtype
    x = harness.tok_dev(inp["x"], tok)
    ids = harness.to_dev(inp["expert_ids"])
    mask = harness.to_dev(inp.get("mask"))
    w = harness.to_dev(inp["expert_scales"])
    out = cq.dispatch(cfg, x, ids, harness.to_dev(inp.get("scales")), mask, expert_scales=w)
    es_ref = oracle.expand_scales(ocfg, ref["assist_info"], ref["recv_offsets"],
                                  inp["expert_scales"], wl.cap)
    eo = workloads.f32_to_tok_bits(np.random.default_rng(seed + 3).standard_normal(
        (wl.cap, wl.H)).astype(np.float32), tok)
    shared = _shared(wl, seed + 4) if with_shared else None
    y_ref = oracle.combine_scatter(ocfg, eo, ref["assist_info"], ref["recv_offsets"],
                                   inp["expert_ids"], inp["expert_scales"],
                                   mask=inp.get("mask"), ori_x=inp["x"], shared_x=shared)
    y = cq.combine_scatter(cfg, harness.tok_dev(eo, tok), out["assist_info"], out["recv_offsets"],
                           ids, w, mask, x, harness.tok_dev(shared, tok) if with_shared else None,
                           workspace=workspace)
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)
    P = int(ref["recv_offsets"][-1])
    np.testing.assert_array_equal(harness.host(out["expand_scales"])[:P].view(np.uint32),
                                  es_ref[:P].view(np.uint32), err_msg="expand_scales")
    return harness.check_combine_tolerance(harness.host(y), y_ref, token_dtype=tok)


@pytest.mark.parametrize("with_shared", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_scatter_back_roundtrip(name, with_shared):
    assert _run(CASES[name], 0, with_shared) == 0


def test_workspace_reused_across_routings():
    """The slot map is rewritten by every call: a workspace left by another routing (and
    larger config) must not leak into the next result."""
    import torch
    import combine_quant_amd as cq
    big = CASES["special_masked_k16"]
    ws = torch.full((cq.moe_dc_combine_scatter_workspace_bytes(harness.lib_cfg(big)),), 0x7F,
                    dtype=torch.uint8, device="cuda")
    assert _run(big, 1, True, workspace=ws) == 0
    assert _run(CASES["dup_mask1d"], 2, True, workspace=ws) == 0
    assert _run(CASES["c1"], 3, False, workspace=ws) == 0


def test_full_size_with_shared():
    """W=16, BS=512, H=7168, K=8 with a shared expert: every token against the oracle."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C4
    inp = workloads.generate(wl, seed=0)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo_dev = workloads.expert_out_torch(wl, wl.cap, seed=0)
    shared = _shared(wl, 9)
    w = harness.to_dev(inp["expert_scales"])
    y = cq.combine_scatter(cfg, eo_dev, out["assist_info"], out["recv_offsets"],
                           dev_in["ids"], w, shared_x=harness.bf16_dev(shared))
    torch.cuda.synchronize()
    y_ref = oracle.combine_scatter(harness.oracle_cfg(wl), harness.host(eo_dev),
                                   harness.host(out["assist_info"]),
                                   harness.host(out["recv_offsets"]), inp["expert_ids"],
                                   inp["expert_scales"], shared_x=shared)
    assert harness.check_combine_tolerance(harness.host(y), y_ref) == 0
