"""GPU parity of the further quantization variants: static int8 (mode 1), per-token fp8
(mode 2 with E4M3/E5M2 codes), per-128-group fp8 (mode 3), MX with E5M2 elements and E8M0
scale bytes or reciprocal fp32 scales, each with every shape of the scales tensor it allows.  Dispatch outputs are
compared with the CPU oracle bit for bit; combine within 1e-2 relative / 1e-3 absolute.
Cases span several workgroups, ragged tails (H not a multiple of 128 or 32; H = 1030 takes
the element-wise kernel), masks, special experts and duplicate picks."""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

WL = workloads.Workload

VARIANTS = {
    # mode 1: static int8, every scales shape; U(16, 48) coefficients saturate the tails
    "static_scalar": WL("static_scalar", W=4, E=32, BS=60, H=1056, K=6, quant_mode=1,
                        scales_kind=1),
    "static_shared": WL("static_shared", W=4, E=32, BS=60, H=2048, K=8, quant_mode=1,
                        scales_kind=2, zero_expert_num=1, copy_expert_num=1, mask_kind=2,
                        inactive_tokens_per_rank=6),
    "static_per_expert": WL("static_per_expert", W=4, E=16, BS=70, H=1024, K=8,
                            quant_mode=1, scales_kind=3, routing="randint"),
    "static_shared_h1030": WL("static_shared_h1030", W=2, E=8, BS=20, H=1030, K=3,
                              quant_mode=1, scales_kind=2),
    # mode 2 with fp8 codes
    "token_e4m3": WL("token_e4m3", W=4, E=32, BS=64, H=1056, K=6, quant_mode=2, out_dtype=2,
                     outlier_prob=0.02),
    "token_e5m2_scalar": WL("token_e5m2_scalar", W=4, E=32, BS=64, H=2048, K=4,
                            quant_mode=2, out_dtype=3, scales_kind=1),
    "token_e4m3_shared": WL("token_e4m3_shared", W=2, E=16, BS=90, H=1024, K=8,
                            quant_mode=2, out_dtype=2, scales_kind=2, mask_kind=1,
                            inactive_tokens_per_rank=10),
    "token_e5m2_per_expert": WL("token_e5m2_per_expert", W=4, E=32, BS=50, H=1056, K=6,
                                quant_mode=2, out_dtype=3, scales_kind=3),
    "token_int8_shared": WL("token_int8_shared", W=4, E=32, BS=50, H=1024, K=8,
                            quant_mode=2, scales_kind=2),
    "token_e4m3_h1030": WL("token_e4m3_h1030", W=2, E=8, BS=17, H=1030, K=3, quant_mode=2,
                           out_dtype=2, scales_kind=3),
    # mode 3: groups of 128, ragged last group at H = 1056 (32) and 1030 (6)
    "group_e4m3": WL("group_e4m3", W=4, E=32, BS=64, H=1056, K=6, quant_mode=3,
                     outlier_prob=0.02),
    "group_e5m2_shared": WL("group_e5m2_shared", W=4, E=32, BS=40, H=2048, K=8,
                            quant_mode=3, out_dtype=3, scales_kind=2),
    "group_e4m3_per_expert": WL("group_e4m3_per_expert", W=4, E=16, BS=60, H=1152, K=16,
                                quant_mode=3, scales_kind=3, routing="randint"),
    "group_e5m2_scalar_special": WL("group_e5m2_scalar_special", W=4, E=32, BS=50, H=1024,
                                    K=8, quant_mode=3, out_dtype=3, scales_kind=1,
                                    zero_expert_num=2, copy_expert_num=2, mask_kind=2,
                                    inactive_tokens_per_rank=5),
    "group_h1030": WL("group_h1030", W=2, E=8, BS=20, H=1030, K=3, quant_mode=3,
                      scales_kind=3),
    "group_h1030_shared": WL("group_h1030_shared", W=2, E=8, BS=20, H=1030, K=2,
                             quant_mode=3, out_dtype=3, scales_kind=2),
    # MX with E5M2 elements and/or E8M0 scale bytes (odd block counts leave a pad slot)
    "mx_e5m2": WL("mx_e5m2", W=3, E=12, BS=77, H=1032, K=5, quant_mode=4, out_dtype=3,
                  routing="zipf"),
    "mx_e4m3_e8m0": WL("mx_e4m3_e8m0", W=4, E=32, BS=60, H=1056, K=6, quant_mode=4,
                       scale_format=1),
    "mxclip_e5m2_e8m0": WL("mxclip_e5m2_e8m0", W=4, E=64, BS=70, H=2048, K=16, quant_mode=5,
                           out_dtype=3, scale_format=1, zero_expert_num=2, copy_expert_num=2,
                           mask_kind=2, inactive_tokens_per_rank=7),
    "mxclip_e5m2": WL("mxclip_e5m2", W=2, E=8, BS=40, H=1056, K=2, quant_mode=5, out_dtype=3),
    "mx_e8m0_h1030": WL("mx_e8m0_h1030", W=2, E=8, BS=33, H=1030, K=3, quant_mode=4,
                        scale_format=1),
    "mxclip_e5m2_e8m0_h1030": WL("mxclip_e5m2_e8m0_h1030", W=2, E=8, BS=33, H=1030, K=3,
                                 quant_mode=5, out_dtype=3, scale_format=1),
    # MX with E2M1 (fp4) elements, two codes per byte
    "mx_e2m1": WL("mx_e2m1", W=3, E=12, BS=77, H=1032, K=5, quant_mode=4, out_dtype=4,
                  routing="zipf"),
    "mxclip_e2m1_e8m0_special": WL("mxclip_e2m1_e8m0_special", W=4, E=64, BS=70, H=2048,
                                   K=16, quant_mode=5, out_dtype=4, scale_format=1,
                                   zero_expert_num=2, copy_expert_num=2, mask_kind=2,
                                   inactive_tokens_per_rank=7),
    # even vector count (8-byte paired stores) with a ragged last wave: 130 vectors
    "mxclip_e2m1_e8m0_h1040": WL("mxclip_e2m1_e8m0_h1040", W=3, E=12, BS=45, H=1040, K=4,
                                 quant_mode=5, out_dtype=4, scale_format=1),
    "mx_e2m1_h1030": WL("mx_e2m1_h1030", W=2, E=8, BS=33, H=1030, K=3, quant_mode=4,
                        out_dtype=4),
    "mxclip_e2m1_h1030": WL("mxclip_e2m1_h1030", W=2, E=8, BS=33, H=1030, K=3,
                            quant_mode=5, out_dtype=4, scale_format=1),
    # MX with reciprocal fp32 scales (2^-shared_exp): tile kernel with a pad slot, special
    # experts and per-pick masks, and the element-wise kernel
    "mx_e4m3_recip": WL("mx_e4m3_recip", W=4, E=32, BS=60, H=1056, K=6, quant_mode=4,
                        scale_format=2),
    "mxclip_e2m1_recip_special": WL("mxclip_e2m1_recip_special", W=4, E=64, BS=70, H=2048,
                                    K=16, quant_mode=5, out_dtype=4, scale_format=2,
                                    zero_expert_num=2, copy_expert_num=2, mask_kind=2,
                                    inactive_tokens_per_rank=7),
    "mxclip_e5m2_recip_h1030": WL("mxclip_e5m2_recip_h1030", W=2, E=8, BS=33, H=1030, K=3,
                                  quant_mode=5, out_dtype=3, scale_format=2),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_variant_roundtrip(name):
    ndiff = harness.roundtrip(VARIANTS[name])
    assert ndiff == 0, f"{ndiff} bf16 elements differ from the oracle (within tolerance)"


@pytest.mark.parametrize("variant", [(2, 1), (2, 2), (2, 3), (3, 2), (3, 3)])
@pytest.mark.parametrize("H", [1024, 1030])
def test_zero_tokens_and_groups(variant, H):
    """All-zero tokens (mode 2) and all-zero 128-groups (mode 3) give codes 0 and scale 0;
    tiny and huge magnitudes sit next to them."""
    import torch
    import combine_quant_amd as cq
    mode, odt = variant
    W, BS = 2, 24
    rng = np.random.default_rng(H + mode)
    xf = rng.standard_normal((W, BS, H)).astype(np.float32)
    xf[:, ::3] = 0.0                                    # whole tokens
    for g in range(0, H, 256):
        xf[:, 1::3, g:g + 128] = 0.0                    # every other group
    xf[:, 2::6] *= np.float32(1e-30)
    xf[:, 5::6] *= np.float32(1e30)
    x = workloads.f32_to_bf16_bits(xf)
    wl = WL("zeros", W=W, E=4, BS=BS, H=H, K=2, quant_mode=mode, out_dtype=odt)
    ids = np.tile(np.array([0, 3], np.int32), (W, BS, 1))
    inp = dict(x=x, expert_ids=ids)
    _, ref = harness.oracle_dispatch(wl, inp)
    out = cq.dispatch(harness.lib_cfg(wl), harness.bf16_dev(x), harness.to_dev(ids))
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)


@pytest.mark.parametrize("mode", [2, 3, 4, 5])
def test_exhaustive_e5m2_via_rows(mode):
    """All finite bf16 patterns as token elements, coded as E5M2 under each fp8 mode."""
    import torch
    import combine_quant_amd as cq
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(b)
    b = b[np.isfinite(f)]
    b = np.random.default_rng(mode).permutation(b)
    H = 1024
    n_tok = (len(b) + H - 1) // H
    x = np.concatenate([b, np.zeros(n_tok * H - len(b), np.uint16)]).reshape(1, n_tok, H)
    x = np.ascontiguousarray(np.concatenate([x, x[:, ::-1]], axis=0))
    wl = WL("e5m2_sweep", W=2, E=2, BS=n_tok, H=H, K=1, quant_mode=mode, out_dtype=3)
    ids = np.zeros((2, n_tok, 1), np.int32)
    inp = dict(x=x, expert_ids=ids)
    _, ref = harness.oracle_dispatch(wl, inp)
    out = cq.dispatch(harness.lib_cfg(wl), harness.bf16_dev(x), harness.to_dev(ids))
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)


@pytest.mark.parametrize("mode", [4, 5])
def test_exhaustive_e2m1_via_rows(mode):
    """All finite bf16 patterns as token elements, coded as E2M1 under both MX modes."""
    import torch
    import combine_quant_amd as cq
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(b)
    b = b[np.isfinite(f)]
    b = np.random.default_rng(10 + mode).permutation(b)
    H = 1024
    n_tok = (len(b) + H - 1) // H
    x = np.concatenate([b, np.zeros(n_tok * H - len(b), np.uint16)]).reshape(1, n_tok, H)
    x = np.ascontiguousarray(np.concatenate([x, x[:, ::-1]], axis=0))
    wl = WL("e2m1_sweep", W=2, E=2, BS=n_tok, H=H, K=1, quant_mode=mode, out_dtype=4)
    ids = np.zeros((2, n_tok, 1), np.int32)
    inp = dict(x=x, expert_ids=ids)
    _, ref = harness.oracle_dispatch(wl, inp)
    out = cq.dispatch(harness.lib_cfg(wl), harness.bf16_dev(x), harness.to_dev(ids))
    torch.cuda.synchronize()
    harness.compare_dispatch(wl, inp, out, ref)


def test_e8m0_bytes_are_the_fp32_exponents():
    """Same input under fp32 and E8M0 scale storage: every byte is the exponent field of the
    fp32 scale (the fp32 2^-127 is subnormal: byte 0), pad bytes 0."""
    import torch
    import combine_quant_amd as cq
    wl = VARIANTS["mx_e4m3_e8m0"]
    inp = workloads.generate(wl, seed=2)
    _, _, a = harness.gpu_dispatch(wl.replace(scale_format=0), inp)
    _, _, b = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    P = int(a["recv_offsets"][-1].item())
    s32 = harness.host(a["dynamic_scales"])[:P]
    s8 = harness.host(b["dynamic_scales"])[:P]
    nb = (wl.H + 31) // 32
    expo = (s32.view(np.uint32) >> 23).astype(np.int64)
    expo[s32.view(np.uint32) == 0x00400000] = 0
    assert (s8[:, :nb] == expo[:, :nb]).all()
    assert (s8[:, nb:] == 0).all()
    assert torch.equal(a["expand_x"][:P], b["expand_x"][:P])
    assert oracle.e8m0_from_scale(2.0 ** -127) == 0


@pytest.mark.parametrize("name", ["mx_e4m3_recip", "mxclip_e5m2_recip_h1030"])
def test_reciprocal_scales_invert_the_fp32_scales(name):
    """Same input under fp32 2^shared_exp and reciprocal scale storage: the codes are the
    same, each product of the two scales is exactly 1 (2^-127 * 2^127 included), pads 0."""
    import torch
    wl = VARIANTS[name]
    inp = workloads.generate(wl, seed=3)
    _, _, a = harness.gpu_dispatch(wl.replace(scale_format=0), inp)
    _, _, b = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    P = int(a["recv_offsets"][-1].item())
    nb = (wl.H + 31) // 32
    sa = harness.host(a["dynamic_scales"])[:P].astype(np.float64)
    sb = harness.host(b["dynamic_scales"])[:P].astype(np.float64)
    assert (sa[:, :nb] * sb[:, :nb] == 1.0).all()
    assert (sb[:, nb:] == 0).all()
    assert torch.equal(a["expand_x"][:P], b["expand_x"][:P])
