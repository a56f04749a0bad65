"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every function
include/moe_dc.h declares, and its host validation enforces the pages' attribute rules."""
import ctypes
import os
import re

import pytest

import combine_quant_amd as cq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dc.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(cq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = cq.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # the exported symbols are plain C names (no C++ mangling)
    raw = ctypes.CDLL(lib._name)
    for name in _declared_functions():
        getattr(raw, name)


def test_config_struct_layout_matches_header():
    # sixteen int32 fields (flags, then token_dtype) then one int64
    assert ctypes.sizeof(cq.MoeDcConfig) == 16 * 4 + 8
    assert cq.MoeDcConfig.out_dtype.offset == 44
    assert cq.MoeDcConfig.scales_kind.offset == 48
    assert cq.MoeDcConfig.scale_format.offset == 52
    assert cq.MoeDcConfig.flags.offset == 56
    assert cq.MoeDcConfig.token_dtype.offset == 60
    assert cq.MoeDcConfig.expand_rows_capacity.offset == 64


def test_header_enum_values_match_the_binding():
    text = open(HEADER).read()
    for name in ("MOE_DTYPE_DEFAULT", "MOE_DTYPE_INT8", "MOE_DTYPE_E4M3", "MOE_DTYPE_E5M2",
                 "MOE_DTYPE_E2M1",
                 "MOE_SCALES_NONE", "MOE_SCALES_SCALAR", "MOE_SCALES_SHARED",
                 "MOE_SCALES_PER_EXPERT", "MOE_SCALE_FP32", "MOE_SCALE_E8M0", "MOE_SCALE_FP32_RECIPROCAL",
                 "MOE_DC_FLAG_SEPARATE_ROUTE", "MOE_DC_FLAG_CHECK_IDS", "MOE_TOKEN_BF16",
                 "MOE_TOKEN_F16"):
        m = re.search(r"\b" + name + r"\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(cq, name), name


def _cfg(**kw):
    base = dict(W=16, E=256, BS=512, H=7168, K=8, quant_mode=2)
    base.update({k: v for k, v in kw.items() if k in base})
    c = cq.make_config(base["W"], base["E"], base["BS"], base["H"], base["K"],
                       base["quant_mode"])
    for k, v in kw.items():
        if k not in base:
            setattr(c, k, v)
    return c


def test_valid_configs_of_the_workloads():
    import workloads
    for wl in workloads.WORKLOADS.values():
        c = cq.make_config(wl.W, wl.E, wl.BS, wl.H, wl.K, wl.quant_mode,
                           zero_expert_num=wl.zero_expert_num,
                           copy_expert_num=wl.copy_expert_num, mask_kind=wl.mask_kind,
                           out_dtype=wl.out_dtype, scales_kind=wl.scales_kind,
                           scale_format=wl.scale_format)
        assert cq.moe_dc_validate(c) == cq.MOE_OK, (wl.name, cq.moe_dc_last_error())


@pytest.mark.parametrize("kw,status", [
    (dict(W=1), cq.MOE_ERR_INVALID_ARG),
    (dict(W=769, E=769), cq.MOE_ERR_INVALID_ARG),
    (dict(E=0), cq.MOE_ERR_INVALID_ARG),
    (dict(E=1040, W=16), cq.MOE_ERR_INVALID_ARG),
    (dict(E=250), cq.MOE_ERR_INVALID_ARG),            # not a multiple of W
    (dict(BS=0), cq.MOE_ERR_INVALID_ARG),
    (dict(BS=513), cq.MOE_ERR_INVALID_ARG),
    (dict(H=1023), cq.MOE_ERR_INVALID_ARG),
    (dict(H=8193), cq.MOE_ERR_INVALID_ARG),
    (dict(K=0), cq.MOE_ERR_INVALID_ARG),
    (dict(K=17), cq.MOE_ERR_INVALID_ARG),
    (dict(W=2, E=2, K=3), cq.MOE_ERR_INVALID_ARG),    # K > number of experts
    (dict(quant_mode=1), cq.MOE_ERR_INVALID_ARG),     # static quant without scales
    (dict(quant_mode=6), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=-1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=0, out_dtype=1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=1, out_dtype=2, scales_kind=1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=3, out_dtype=1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=4, out_dtype=1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=2, out_dtype=4), cq.MOE_ERR_INVALID_ARG),      # fp4 only for MX
    (dict(quant_mode=3, out_dtype=4), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=4, out_dtype=4, H=1025), cq.MOE_ERR_INVALID_ARG),  # fp4 needs even H
    (dict(quant_mode=5, out_dtype=5), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=4, scales_kind=2), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=0, scales_kind=1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=2, scales_kind=4), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=2, scale_format=1), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=5, scale_format=3), cq.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=3, scale_format=2), cq.MOE_ERR_INVALID_ARG),   # reciprocal: MX only
    (dict(const_expert_num=1), cq.MOE_ERR_UNSUPPORTED),
    (dict(zero_expert_num=-1), cq.MOE_ERR_INVALID_ARG),
    (dict(zero_expert_num=2 ** 31 - 100), cq.MOE_ERR_INVALID_ARG),   # id space >= INT32_MAX
    (dict(expert_token_nums_type=2), cq.MOE_ERR_INVALID_ARG),
    (dict(mask_kind=3), cq.MOE_ERR_INVALID_ARG),
    (dict(token_dtype=2), cq.MOE_ERR_INVALID_ARG),
    (dict(token_dtype=-1), cq.MOE_ERR_INVALID_ARG),
    (dict(flags=4), cq.MOE_ERR_INVALID_ARG),
    (dict(flags=-1), cq.MOE_ERR_INVALID_ARG),
    (dict(expand_rows_capacity=16 * 512 * 8 - 1), cq.MOE_ERR_INVALID_ARG),
    (dict(expand_rows_capacity=2 ** 31), cq.MOE_ERR_INVALID_ARG),
])
def test_validation_rules(kw, status):
    c = _cfg(**kw)
    assert cq.moe_dc_validate(c) == status
    assert cq.moe_dc_last_error() != ""
    assert cq.moe_dc_dispatch_workspace_bytes(c) == 0
    assert cq.moe_dc_scales_per_row(c) == -1


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_known_flags_are_valid(flags):
    c = _cfg(flags=flags)
    assert cq.moe_dc_validate(c) == cq.MOE_OK, cq.moe_dc_last_error()


def test_workspace_holds_the_checked_ids_word_and_per_rank_counts():
    # 256 bytes for the checked-ids word, then the (expert, source) counts and W per-rank
    # counts, each rounded up to 256 bytes
    c = _cfg(W=16, E=256)
    assert cq.moe_dc_dispatch_workspace_bytes(c) == 256 + 256 * 16 * 4 + 256
    c = _cfg(W=3, E=9, BS=5)
    assert cq.moe_dc_dispatch_workspace_bytes(c) == 256 + 256 + 256
    # more than 16,384 counts: the two-launch scan also keeps one total per group of ranks
    # (at most W of them)
    c = _cfg(W=768, E=768, BS=4, H=1024, K=2)
    assert cq.moe_dc_dispatch_workspace_bytes(c) == 256 + 768 * 768 * 4 + 3072 + 3072


def test_k_may_count_special_experts():
    c = _cfg(W=2, E=2, K=4, zero_expert_num=1, copy_expert_num=1)
    assert cq.moe_dc_validate(c) == cq.MOE_OK


@pytest.mark.parametrize("kw", [
    dict(quant_mode=1, scales_kind=1), dict(quant_mode=1, out_dtype=1, scales_kind=3),
    dict(quant_mode=2, out_dtype=2, scales_kind=2), dict(quant_mode=2, out_dtype=3),
    dict(quant_mode=3), dict(quant_mode=3, out_dtype=3, scales_kind=3),
    dict(quant_mode=4, out_dtype=3, scale_format=1), dict(quant_mode=5, scale_format=1),
    dict(quant_mode=4, out_dtype=4), dict(quant_mode=5, out_dtype=4, scale_format=1, H=1030),
    dict(quant_mode=4, scale_format=2), dict(quant_mode=5, out_dtype=4, scale_format=2),
])
def test_quant_variants_validate(kw):
    assert cq.moe_dc_validate(_cfg(**kw)) == cq.MOE_OK, cq.moe_dc_last_error()


def test_scales_per_row_and_workspace():
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=0)) == 0
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=1, scales_kind=1)) == 0
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=2)) == 1
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=3)) == 56         # 7168/128
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=3, H=1030)) == 9   # ceil(1030/128)
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=4)) == 224        # 7168/32, even
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=5, H=1056)) == 34  # 33 blocks -> 34
    assert cq.moe_dc_scales_per_row(_cfg(quant_mode=4, H=1030)) == 34  # ceil(1030/32)=33
    ws = cq.moe_dc_dispatch_workspace_bytes(_cfg())
    assert ws >= 256 * 16 * 4 and ws % 256 == 0


def _dispatch_raw(lib, cfg, x=None, ids=None, scales=None, mask=None, weights=None,
                  expand_x=None, dyn=None, eidx=None, assist=None, erc=None, etn=None,
                  roff=None, expand_scales=None, ws=None, ws_bytes=0):
    return lib.moe_dispatch(ctypes.byref(cfg), x, ids, scales, mask, weights, expand_x, dyn,
                            eidx, assist, erc, etn, roff, expand_scales, ws,
                            ctypes.c_size_t(ws_bytes), None)


def test_dispatch_rejects_bad_arguments_before_any_device_work():
    """Argument errors return a status without touching the device (null pointers)."""
    lib = cq.load_library()
    c = _cfg()
    assert _dispatch_raw(lib, c) == cq.MOE_ERR_INVALID_ARG
    assert "NULL" in cq.moe_dc_last_error()
    rc = lib.moe_combine(ctypes.byref(c), *([None] * 9), None)
    assert rc == cq.MOE_ERR_INVALID_ARG
    rc = lib.moe_combine_scatter(ctypes.byref(c), *([None] * 10), ctypes.c_size_t(0), None)
    assert rc == cq.MOE_ERR_INVALID_ARG
    rc = lib.moe_combine_quantize(ctypes.byref(c), *([None] * 4), None)
    assert rc == cq.MOE_ERR_INVALID_ARG
    rc = lib.moe_combine_int8(ctypes.byref(c), *([None] * 10), None)
    assert rc == cq.MOE_ERR_INVALID_ARG
    assert _dispatch_raw(lib, _cfg(const_expert_num=1)) == cq.MOE_ERR_UNSUPPORTED


def test_dispatch_workspace_and_mask_rules_on_host():
    """With non-null dummy pointers the remaining host rules still fire before any launch."""
    lib = cq.load_library()
    p = ctypes.c_void_p(0x1000)
    full = dict(x=p, ids=p, expand_x=p, dyn=p, eidx=p, assist=p, erc=p, etn=p, roff=p, ws=p,
                ws_bytes=1 << 20)
    c = _cfg()
    # a scales tensor the config does not announce, and a missing one it does
    rc = _dispatch_raw(lib, _cfg(quant_mode=4), scales=p, **full)
    assert rc == cq.MOE_ERR_INVALID_ARG and "scales" in cq.moe_dc_last_error()
    rc = _dispatch_raw(lib, _cfg(quant_mode=1, scales_kind=2), **dict(full, dyn=None))
    assert rc == cq.MOE_ERR_INVALID_ARG and "scales" in cq.moe_dc_last_error()
    # mode 3 needs dynamic_scales
    rc = _dispatch_raw(lib, _cfg(quant_mode=3), **dict(full, dyn=None))
    assert rc == cq.MOE_ERR_INVALID_ARG and "dynamic_scales" in cq.moe_dc_last_error()
    # mask pointer without a mask kind
    rc = _dispatch_raw(lib, c, mask=p, **full)
    assert rc == cq.MOE_ERR_INVALID_ARG and "mask" in cq.moe_dc_last_error()
    # expert_scales without expand_scales
    rc = _dispatch_raw(lib, c, weights=p, **full)
    assert rc == cq.MOE_ERR_INVALID_ARG and "expand_scales" in cq.moe_dc_last_error()
    # workspace too small, and misaligned
    rc = _dispatch_raw(lib, c, **dict(full, ws_bytes=8))
    assert rc == cq.MOE_ERR_WORKSPACE
    rc = _dispatch_raw(lib, c, **dict(full, ws=ctypes.c_void_p(0x1002)))
    assert rc == cq.MOE_ERR_INVALID_ARG and "aligned" in cq.moe_dc_last_error()
    # combine: copy experts without ori_x
    cc = _cfg(copy_expert_num=1)
    rc = lib.moe_combine(ctypes.byref(cc), p, p, p, p, p, p, None, None, p, None)
    assert rc == cq.MOE_ERR_INVALID_ARG and "ori_x" in cq.moe_dc_last_error()
    # scatter-back combine: workspace rules
    need = cq.moe_dc_combine_scatter_workspace_bytes(c)
    assert need == 16 * 512 * 8 * 4
    rc = lib.moe_combine_scatter(ctypes.byref(c), p, p, p, p, p, None, None, None, p, p,
                                 ctypes.c_size_t(need - 1), None)
    assert rc == cq.MOE_ERR_WORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch
    c = _cfg(W=2, E=8, BS=16, H=1024, K=2)
    x = torch.zeros((2, 16, 1024), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cq.moe_dispatch(c, x, None, None, None, None, None, None, None, None, None, None, None)
    with pytest.raises(ValueError):
        cq.moe_combine_scatter(c, x, None, None, None, None, None, None, None, x, None)
