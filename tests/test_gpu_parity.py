"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, same seeded inputs.

Dispatch outputs must match bit for bit (counts, indices, offsets, rows, codes, scales);
combine must be within 1e-2 relative / 1e-3 absolute per bf16 element of the oracle (and
is observed to be bit-identical, which a separate test records).
"""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

W2 = workloads.C1_MODE0

# small cases the oracle finishes in well under a second, covering several workgroups,
# ragged tails (BS not a multiple of 32-token words, H not a multiple of 256 / 32 / 8),
# masks, special experts and duplicate picks
SMALL = {
    "c1_mode0": workloads.C1_MODE0,
    "c1_mode2": workloads.C1_MODE2,
    "c1_mode4": workloads.C1_MODE0.replace(name="c1_mode4", quant_mode=4),
    "c1_mode5": workloads.C1_MODE0.replace(name="c1_mode5", quant_mode=5),
    "smooth_ragged": workloads.Workload("smooth_ragged", W=4, E=32, BS=100, H=1056, K=6,
                                        quant_mode=2, scales_kind=3, outlier_prob=0.02,
                                        expert_token_nums_type=0),
    "mx_ragged_blocks": workloads.Workload("mx_ragged_blocks", W=3, E=12, BS=77, H=1032, K=5,
                                           quant_mode=4, routing="zipf"),
    "mxclip_masked_special": workloads.Workload(
        "mxclip_masked_special", W=4, E=64, BS=70, H=2048, K=16, quant_mode=5,
        zero_expert_num=2, copy_expert_num=2, mask_kind=2, inactive_tokens_per_rank=7),
    "dup_picks_mask1d": workloads.Workload("dup_picks_mask1d", W=2, E=4, BS=65, H=1024, K=6,
                                           quant_mode=2, routing="randint", zero_expert_num=1,
                                           copy_expert_num=1, mask_kind=1,
                                           inactive_tokens_per_rank=9),
    "dup_picks_k16": workloads.Workload("dup_picks_k16", W=4, E=16, BS=140, H=1024, K=16,
                                        quant_mode=4, routing="randint"),
    "scalar_path_h1030": workloads.Workload("scalar_path_h1030", W=2, E=8, BS=33, H=1030, K=3,
                                            quant_mode=5),
    "scalar_path_mode2_h1030": workloads.Workload("scalar_path_mode2_h1030", W=2, E=8, BS=9,
                                                  H=1030, K=3, quant_mode=2, scales_kind=3),
    "scalar_path_mode0_h1030": workloads.Workload("scalar_path_mode0_h1030", W=3, E=9, BS=9,
                                                  H=1030, K=2, quant_mode=0, copy_expert_num=1),
    "l1_w8_k8": workloads.Workload("l1_w8_k8", W=8, E=8, BS=40, H=1024, K=8, quant_mode=4),
    "vec_ids_k8_special": workloads.Workload("vec_ids_k8_special", W=4, E=32, BS=50, H=1024, K=8,
                                             quant_mode=2, zero_expert_num=1,
                                             copy_expert_num=1, mask_kind=1,
                                             inactive_tokens_per_rank=5),
    "vec_ids_k4_special": workloads.Workload("vec_ids_k4_special", W=2, E=16, BS=90, H=1024, K=4,
                                             quant_mode=4, zero_expert_num=2,
                                             copy_expert_num=1, mask_kind=2,
                                             inactive_tokens_per_rank=4),
    "bs1_h8192": workloads.Workload("bs1_h8192", W=2, E=2, BS=1, H=8192, K=2, quant_mode=2),
    "w768_e768": workloads.Workload("w768_e768", W=768, E=768, BS=1, H=1024, K=2,
                                    quant_mode=2),
    # per-expert scales with the separate routing (flags 1): one workgroup per pick, a token
    # count that is not a multiple of 8 (the XCD placement groups tokens by 8), K = 16, a ragged
    # row (the second of two waves holds one vector) and the widest row (four waves of four
    # slots)
    "pick_group_k16_ragged": workloads.Workload("pick_group_k16_ragged", W=3, E=48, BS=37,
                                                H=1032, K=16, quant_mode=3, scales_kind=3),
    "pick_static_h8192": workloads.Workload("pick_static_h8192", W=2, E=8, BS=9, H=8192, K=4,
                                            quant_mode=1, scales_kind=3),
    "pick_token_e5m2_w8": workloads.Workload("pick_token_e5m2_w8", W=8, E=64, BS=65, H=7168,
                                             K=8, quant_mode=2, out_dtype=3, scales_kind=3,
                                             mask_kind=2, inactive_tokens_per_rank=5),
    # the pick kernel's two expert groups with very few experts: one expert per group (and a
    # zero expert), and groups of two and one (and a copy expert)
    "pick_groups_two_experts": workloads.Workload(
        "pick_groups_two_experts", W=2, E=2, BS=512, H=1056, K=3, quant_mode=3, out_dtype=3,
        scales_kind=3, zero_expert_num=1, routing="randint"),
    "pick_groups_three_experts": workloads.Workload(
        "pick_groups_three_experts", W=3, E=3, BS=400, H=2048, K=3, quant_mode=2,
        scales_kind=3, copy_expert_num=1, mask_kind=1, inactive_tokens_per_rank=17),
    # more (expert, source) counts than one LDS pass of the scan holds: chunked scan, with a
    # short last chunk (24,192 counts) and with whole chunks (65,536 counts)
    "scan_chunks_w24_e1008": workloads.Workload("scan_chunks_w24_e1008", W=24, E=1008, BS=8,
                                                H=1024, K=4, quant_mode=2,
                                                expert_token_nums_type=0),
    "scan_chunks_w64_e1024": workloads.Workload("scan_chunks_w64_e1024", W=64, E=1024, BS=4,
                                                H=1024, K=8, quant_mode=4, zero_expert_num=1,
                                                mask_kind=2, inactive_tokens_per_rank=1),
    # per-expert scales past the pick-kernel limit (32,768 picks: a workgroup per window of 256
    # tokens and expert, the window's picks of the expert one after another) with rows that
    # end inside a wave's slots, so lanes past the end read zeros and drop their stores; every
    # mode that takes per-expert scales
    "tile_per_expert_token_ragged": workloads.Workload(
        "tile_per_expert_token_ragged", W=4, E=32, BS=512, H=1056, K=16, quant_mode=2,
        scales_kind=3, outlier_prob=0.02),
    "tile_per_expert_group_ragged": workloads.Workload(
        "tile_per_expert_group_ragged", W=4, E=32, BS=512, H=1160, K=16, quant_mode=3,
        out_dtype=2, scales_kind=3, mask_kind=2, inactive_tokens_per_rank=9),
    "tile_per_expert_static_ragged": workloads.Workload(
        "tile_per_expert_static_ragged", W=4, E=32, BS=512, H=2056, K=16, quant_mode=1,
        scales_kind=3),
    # 12,288 picks at the c2 row shape: one workgroup per pick and expert group
    "pick_12k_picks_h7168": workloads.Workload(
        "pick_12k_picks_h7168", W=8, E=256, BS=192, H=7168, K=8, quant_mode=2,
        scales_kind=3, outlier_prob=0.01),
    # just past the pick kernel's limit (17,408 picks): 272-token windows at the c2 row shape
    "window_17k_picks_h7168": workloads.Workload(
        "window_17k_picks_h7168", W=8, E=256, BS=272, H=7168, K=8, quant_mode=2,
        scales_kind=3, outlier_prob=0.01),
    # windows that span source ranks (BS=23, 288-token windows, the last one shorter), masks
    # and special experts
    "window_spans_ranks_masked": workloads.Workload(
        "window_spans_ranks_masked", W=100, E=200, BS=23, H=1096, K=8, quant_mode=2,
        scales_kind=3, mask_kind=2, inactive_tokens_per_rank=3, zero_expert_num=1,
        copy_expert_num=1),
    # ids drawn with repetition over 16 experts: a token lists an expert several times, so a
    # window's list holds up to K entries per token
    "window_repeated_ids_group": workloads.Workload(
        "window_repeated_ids_group", W=8, E=16, BS=512, H=1024, K=8, quant_mode=3,
        out_dtype=3, scales_kind=3, routing="randint"),
    # the widest row in windows (eight waves, no spare maximum slots) with per-token E4M3
    # codes, and static int8 codes on per-expert coefficients
    "window_h8192_e4m3": workloads.Workload(
        "window_h8192_e4m3", W=8, E=64, BS=512, H=8192, K=8, quant_mode=2, out_dtype=2,
        scales_kind=3, outlier_prob=0.01),
    "window_h8192_static": workloads.Workload(
        "window_h8192_static", W=8, E=64, BS=512, H=8192, K=8, quant_mode=1, scales_kind=3),
    # too many experts for the windows (512-token windows at K=2 would average one pick per
    # expert): token workgroups, their picks one after another
    "token_per_expert_e1024": workloads.Workload(
        "token_per_expert_e1024", W=32, E=1024, BS=512, H=1024, K=2, quant_mode=2,
        scales_kind=3),
}


_oracle_dispatch = harness.oracle_dispatch
_roundtrip = harness.roundtrip


@pytest.mark.parametrize("flags", [0, 1])     # 1: MOE_DC_FLAG_SEPARATE_ROUTE
@pytest.mark.parametrize("name", list(SMALL))
def test_small_roundtrip(name, flags):
    ndiff = _roundtrip(SMALL[name], flags=flags)
    assert ndiff == 0, f"{ndiff} bf16 elements differ from the oracle (within tolerance)"


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_c1_seeds(seed):
    for wl in (workloads.C1_MODE0, workloads.C1_MODE2):
        assert _roundtrip(wl, seed) == 0


def test_c2_full_both_etn_types():
    """W=8, BS=128, H=7168, K=8 with smooth scales and outliers: every output compared."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C2
    inp = workloads.generate(wl, seed=0)
    for etn in (0, 1):
        w = wl.replace(expert_token_nums_type=etn)
        ocfg, ref = _oracle_dispatch(w, inp)
        cfg, dev_in, out = harness.gpu_dispatch(w, inp)
        torch.cuda.synchronize()
        harness.compare_dispatch(w, inp, out, ref)
    # identity-dequant FFN round trip: expert_out = bf16(q * scale) on both sides
    P = int(ref["recv_offsets"][-1])
    deq = ref["expand_x"].astype(np.float32) * ref["dynamic_scales"][:, None]
    eo_ref = workloads.f32_to_bf16_bits(deq)
    y_ref = oracle.combine(ocfg, eo_ref, inp["expert_ids"], ref["expand_idx"],
                           inp["expert_scales"], ref["ep_recv_count"], ref["recv_offsets"])
    eo = (out["expand_x"].float() * out["dynamic_scales"][:, None]).to(torch.bfloat16)
    y = cq.combine(cfg, eo, dev_in["ids"], out["expand_idx"],
                   harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                   out["recv_offsets"])
    torch.cuda.synchronize()
    assert P == wl.cap
    assert harness.check_combine_tolerance(harness.host(y), y_ref) == 0


def test_determinism_repeat():
    import torch
    wl = SMALL["mxclip_masked_special"]
    inp = workloads.generate(wl, seed=5)
    _, _, a = harness.gpu_dispatch(wl, inp)
    _, _, b = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    for k in a:
        if k == "workspace" or a[k] is None:
            continue
        P = int(a["recv_offsets"][-1].item())
        ta, tb = (a[k][:P], b[k][:P]) if k in ("expand_x", "dynamic_scales",
                                               "assist_info") else (a[k], b[k])
        assert torch.equal(ta, tb), k


@pytest.mark.parametrize("flags", [0, 1])     # 1: MOE_DC_FLAG_SEPARATE_ROUTE
def test_all_tokens_inactive(flags):
    import torch
    import combine_quant_amd as cq
    wl = workloads.Workload("all_off", W=2, E=8, BS=16, H=1024, K=2, quant_mode=2, mask_kind=2,
                            inactive_tokens_per_rank=16, copy_expert_num=1)
    inp = workloads.generate(wl, seed=0)
    assert inp["mask"].sum() == 0
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp, cfg=harness.lib_cfg(wl, flags=flags))
    y = cq.combine(cfg, torch.zeros((wl.cap, wl.H), dtype=torch.bfloat16, device="cuda"),
                   dev_in["ids"], out["expand_idx"], harness.to_dev(inp["expert_scales"]),
                   out["ep_recv_count"], out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    assert (harness.host(out["expand_idx"]) == -1).all()
    assert (harness.host(out["ep_recv_count"]) == 0).all()
    assert (harness.host(out["recv_offsets"]) == 0).all()
    assert (harness.host(y) == 0).all()


def test_unaligned_pointers_take_the_scalar_path():
    """x offset by one element: the library must fall back to element-wise kernels and
    still match the oracle."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C1_MODE2.replace(quant_mode=4)
    inp = workloads.generate(wl, seed=3)
    _, ref = _oracle_dispatch(wl, inp)
    cfg = harness.lib_cfg(wl)
    xbuf = torch.empty(inp["x"].size + 1, dtype=torch.bfloat16, device="cuda")
    xbuf[1:] = harness.bf16_dev(inp["x"].ravel())
    x = xbuf[1:].view(wl.W, wl.BS, wl.H)
    assert x.data_ptr() % 16 != 0
    out = cq.dispatch(cfg, x, harness.to_dev(inp["expert_ids"]))
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)


def test_exhaustive_int8_scale_via_rows():
    """Every positive finite bf16 value as a token's absolute maximum (one token each):
    dyn = 127/amax and scale = 1/dyn must round exactly like the oracle's."""
    import torch
    import combine_quant_amd as cq
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    T = len(amax_bits)
    W = 2
    BS = 512
    n_tok = W * BS
    H = 1024
    for lo in range(0, T, n_tok):
        chunk = amax_bits[lo:lo + n_tok]
        x = np.zeros((n_tok, H), np.uint16)
        x[:len(chunk), 0] = chunk
        x[:len(chunk), 1] = chunk | 0x8000          # a negative copy at the same magnitude
        x[:len(chunk), 2] = np.where(chunk > 0x0100, chunk - 0x0100, 0)  # smaller values
        x = x.reshape(W, BS, H)
        ids = np.zeros((W, BS, 1), np.int32)
        wl = workloads.Workload("amax_sweep", W=W, E=2, BS=BS, H=H, K=1, quant_mode=2)
        inp = dict(x=x, expert_ids=ids)
        _, ref = _oracle_dispatch(wl, inp)
        cfg = harness.lib_cfg(wl)
        out = cq.dispatch(cfg, harness.bf16_dev(x), harness.to_dev(ids))
        torch.cuda.synchronize()
        harness.compare_dispatch(wl, inp, out, ref)


def test_exhaustive_e4m3_via_rows():
    """All 65,536 bf16 patterns except NaN/inf, as MX elements under both MX modes, against
    the oracle; blocks mix magnitudes so many shared exponents are exercised."""
    import torch
    import combine_quant_amd as cq
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(b)
    b = b[np.isfinite(f)]
    rng = np.random.default_rng(0)
    b = rng.permutation(b)
    H = 1024
    n_tok = (len(b) + H - 1) // H
    pad = np.zeros(n_tok * H - len(b), np.uint16)
    x = np.concatenate([b, pad]).reshape(1, n_tok, H)
    x = np.concatenate([x, x[:, ::-1]], axis=0)      # W=2
    for mode in (4, 5):
        wl = workloads.Workload("e4m3_sweep", W=2, E=2, BS=n_tok, H=H, K=1, quant_mode=mode)
        ids = np.zeros((2, n_tok, 1), np.int32)
        inp = dict(x=np.ascontiguousarray(x), expert_ids=ids)
        _, ref = _oracle_dispatch(wl, inp)
        out = cq.dispatch(harness.lib_cfg(wl), harness.bf16_dev(inp["x"]), harness.to_dev(ids))
        torch.cuda.synchronize()
        harness.compare_dispatch(wl, inp, out, ref)


def test_invalid_arguments_raise_and_enqueue_nothing():
    import torch
    import combine_quant_amd as cq
    wl = workloads.C1_MODE2
    inp = workloads.generate(wl, seed=0)
    cfg = harness.lib_cfg(wl)
    x = harness.bf16_dev(inp["x"])
    ids = harness.to_dev(inp["expert_ids"])
    o = cq.alloc_dispatch_outputs(cfg)
    o["expand_idx"].fill_(123)
    small_ws = o["workspace"][:8]
    with pytest.raises(cq.MoeDcError) as ei:
        cq.moe_dispatch(cfg, x, ids, None, None, o["expand_x"], o["dynamic_scales"],
                        o["expand_idx"], o["assist_info"], o["ep_recv_count"],
                        o["expert_token_nums"], o["recv_offsets"], small_ws)
    assert ei.value.status == cq.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (o["expand_idx"] == 123).all()


# 1: MOE_DC_FLAG_SEPARATE_ROUTE, 2: MOE_DC_FLAG_CHECK_IDS; the (W, E) pairs give 128 (expert,
# source) counts, and 65,536 (the two-launch scan of wide count matrices)
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("K", [3, 4, 8, 16])
@pytest.mark.parametrize("W,E,BS", [(4, 32, 60), (64, 1024, 6)])
def test_out_of_range_ids_are_not_dispatched(W, E, BS, K, flags):
    """Ids outside [0, E+Z+C) break the contract; the library must treat such picks exactly
    like masked-off picks (no row, expand_idx -1, no combine term) and never touch memory
    out of bounds.  Reference: the oracle on the same input with those picks masked off.
    With the id check, the workspace's first int32 holds the number of active bad picks."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.Workload("bad_ids", W=W, E=E, BS=BS, H=1024, K=K, quant_mode=2,
                            zero_expert_num=1, copy_expert_num=1, mask_kind=2)
    inp = workloads.generate(wl, seed=11)
    rng = np.random.default_rng(5)
    bad = rng.random(inp["expert_ids"].shape) < 0.1
    ids_bad = inp["expert_ids"].copy()
    ids_bad[bad] = rng.choice([-7, -1, wl.n_ids, wl.n_ids + 3, 1 << 30], size=int(bad.sum()))
    # reference: same routing with the bad picks masked off and given a harmless id
    ref_mask = inp["mask"].copy()
    ref_mask[bad] = 0
    ref_ids = ids_bad.copy()
    ref_ids[bad] = 0
    ocfg = harness.oracle_cfg(wl)
    ref = oracle.dispatch(ocfg, inp["x"], ref_ids, mask=ref_mask)
    cfg = harness.lib_cfg(wl, flags=flags)
    x = harness.bf16_dev(inp["x"])
    ids_dev = harness.to_dev(ids_bad)
    mask_dev = harness.to_dev(inp["mask"])
    out = cq.dispatch(cfg, x, ids_dev, None, mask_dev)
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)
    if flags & cq.MOE_DC_FLAG_CHECK_IDS:
        n_bad = int((bad & (inp["mask"] != 0)).sum())
        assert n_bad > 0
        assert int(out["workspace"][:4].view(torch.int32).item()) == n_bad
    rng2 = np.random.default_rng(6)
    eo = workloads.f32_to_bf16_bits(rng2.standard_normal((wl.cap, wl.H), dtype=np.float32))
    y_ref = oracle.combine(ocfg, eo, ref_ids, ref["expand_idx"], inp["expert_scales"],
                           ref["ep_recv_count"], ref["recv_offsets"], mask=ref_mask,
                           ori_x=inp["x"])
    y = cq.combine(cfg, harness.bf16_dev(eo), ids_dev, out["expand_idx"],
                   harness.to_dev(inp["expert_scales"]), out["ep_recv_count"],
                   out["recv_offsets"], mask_dev, x)
    torch.cuda.synchronize()
    assert harness.check_combine_tolerance(harness.host(y), y_ref) == 0
    if flags & cq.MOE_DC_FLAG_CHECK_IDS:
        # a clean batch through the same workspace reports zero
        cq.dispatch(cfg, x, harness.to_dev(ref_ids), None, mask_dev, out=out)
        torch.cuda.synchronize()
        assert int(out["workspace"][:4].view(torch.int32).item()) == 0
